"""ctypes binding of libqd (include/qd.h): the same entry points, argument
marshalling only.  Every step of the decode path runs in the library's HIP
kernels; this module never computes anything itself and raises if the
library is missing.

Device memory and streams come from PyTorch: pass torch tensors (on the GPU)
or raw integer device pointers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqd.so")

QD_OK = 0
QD_EINVAL = -1
QD_EUNSUPPORTED = -2
QD_ESTATE = -3
QD_EHIP = -4
QD_ENOMEM = -5

QD_DEV_BAD_TOKEN = 1
QD_DEV_BAD_POSITION = 2
QD_DEV_BAD_PAGE = 4
QD_DEV_TIMEOUT = 8

EXPORTED = ("qd_create", "qd_load_weights", "qd_decode_step", "qd_prefill", "qd_prefill_prompts",
            "qd_decode_step_taps",
            "qd_stream_step_taps", "qd_read_ceiling", "qd_sample_noalloc",
            "qd_profile_step", "qd_profile_class", "qd_device_status", "qd_stream",
            "qd_step_path", "qd_sample", "qd_destroy", "qd_last_error",
            "qd_blocks_create", "qd_blocks_destroy", "qd_blocks_add", "qd_blocks_reserve",
            "qd_blocks_release", "qd_blocks_fork", "qd_blocks_tables", "qd_blocks_length",
            "qd_blocks_available", "qd_blocks_publish", "qd_blocks_match",
            "qd_engine_create", "qd_engine_destroy", "qd_engine_submit", "qd_engine_step",
            "qd_engine_get_stats")

PROF_CLASSES = ("embed", "qkv", "attention", "o_proj", "gate_up", "down", "lm_head")


class QdConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tie_embeddings", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("page_size", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("use_graphs", ctypes.c_int32), ("persistent", ctypes.c_int32),
                ("max_prefill_rows", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class QdTensorDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 2), ("dtype", ctypes.c_int32)]


class QdTaps(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("x_in", "qkv", "q_rot", "k_rot", "attn", "x_mid", "act",
                                       "x_out", "final_h")]


TAP_NAMES = ("x_in", "qkv", "q_rot", "k_rot", "attn", "x_mid", "act", "x_out", "final_h")

_lib = None


class QdEngineRequest(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int64), ("prompt", ctypes.c_void_p), ("n_prompt", ctypes.c_int32),
                ("max_new_tokens", ctypes.c_int32), ("eos_id", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("seed", ctypes.c_uint64)]


class QdEngineStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("prefill_rows", ctypes.c_int64),
                ("cached_rows", ctypes.c_int64), ("decode_rows", ctypes.c_int64),
                ("tokens_out", ctypes.c_int64), ("sampled_iterations", ctypes.c_int64),
                ("gpu_us", ctypes.c_int64),
                ("waiting", ctypes.c_int32),
                ("running", ctypes.c_int32), ("pages_available", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class QdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qd error {code}: {msg}")
        self.code = code


def load_library():
    """Load libqd.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.qd_create.restype = ctypes.c_int
        lib.qd_create.argtypes = [ctypes.POINTER(QdConfig), P, ctypes.POINTER(P)]
        lib.qd_load_weights.restype = ctypes.c_int
        lib.qd_load_weights.argtypes = [P, ctypes.POINTER(QdTensorDesc), ctypes.c_int32]
        lib.qd_decode_step.restype = ctypes.c_int
        lib.qd_decode_step.argtypes = [P, ctypes.c_int32, P, P, P, P, P, P]
        lib.qd_prefill.restype = ctypes.c_int
        lib.qd_prefill.argtypes = [P, ctypes.c_int32, P, P, P, P, ctypes.c_int32, P, P]
        lib.qd_prefill_prompts.restype = ctypes.c_int
        lib.qd_prefill_prompts.argtypes = [P, ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, P]
        lib.qd_decode_step_taps.restype = ctypes.c_int
        lib.qd_decode_step_taps.argtypes = [P, ctypes.c_int32, P, P, P, P, P, P,
                                            ctypes.POINTER(QdTaps)]
        lib.qd_stream_step_taps.restype = ctypes.c_int
        lib.qd_stream_step_taps.argtypes = [P, P, P, P, P, P, P, ctypes.POINTER(QdTaps)]
        lib.qd_sample_noalloc.restype = ctypes.c_int
        lib.qd_sample_noalloc.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P]
        lib.qd_read_ceiling.restype = ctypes.c_int
        lib.qd_read_ceiling.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P,
                                        ctypes.POINTER(ctypes.c_float)]
        lib.qd_profile_step.restype = ctypes.c_int
        lib.qd_profile_step.argtypes = [P, ctypes.c_int32, P, P, P, P, P, P,
                                        ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_int32)]
        lib.qd_profile_class.restype = ctypes.c_int
        lib.qd_profile_class.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float)]
        I32, I64 = ctypes.c_int32, ctypes.c_int64
        for name, args in (("qd_blocks_create", [I32, I32, ctypes.POINTER(P)]),
                           ("qd_blocks_add", [P, I64]), ("qd_blocks_reserve", [P, I64, I32]),
                           ("qd_blocks_release", [P, I64]), ("qd_blocks_fork", [P, I64, I64, P, P]),
                           ("qd_blocks_tables", [P, P, I32, I32, P]),
                           ("qd_blocks_length", [P, I64]), ("qd_blocks_available", [P]),
                           ("qd_blocks_publish", [P, I64, P, I32]),
                           ("qd_blocks_match", [P, I64, P, I32])):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = args
        lib.qd_blocks_destroy.restype = None
        for name, args in (("qd_engine_create", [P, P, ctypes.POINTER(P)]),
                           ("qd_engine_submit", [P, ctypes.POINTER(QdEngineRequest)]),
                           ("qd_engine_step", [P, I32, P, P, P, ctypes.POINTER(I32)]),
                           ("qd_engine_get_stats", [P, ctypes.POINTER(QdEngineStats)])):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = args
        lib.qd_engine_destroy.restype = None
        lib.qd_engine_destroy.argtypes = [P]
        lib.qd_blocks_destroy.argtypes = [P]
        lib.qd_sample.restype = ctypes.c_int
        lib.qd_sample.argtypes = [P, ctypes.c_int32, P, P, P, P, P, P]
        lib.qd_device_status.restype = ctypes.c_int
        lib.qd_device_status.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
        lib.qd_stream.restype = P
        lib.qd_stream.argtypes = [P]
        lib.qd_step_path.restype = ctypes.c_int
        lib.qd_step_path.argtypes = [P, ctypes.c_int32]
        lib.qd_destroy.restype = None
        lib.qd_destroy.argtypes = [P]
        lib.qd_last_error.restype = ctypes.c_char_p
        lib.qd_last_error.argtypes = [P]
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(rc: int, handle) -> None:
    if rc != QD_OK:
        msg = load_library().qd_last_error(handle)
        raise QdError(rc, msg.decode() if msg else "")


def make_config(shape, max_batch: int, max_pages_per_seq: int, num_pages: int,
                use_graphs: bool = True, persistent: bool = False,
                max_prefill_rows: int = 0, kv_fp8: bool = False, k_scale: float = 1.0,
                v_scale: float = 1.0) -> QdConfig:
    return QdConfig(shape.num_layers, shape.hidden, shape.num_q_heads, shape.num_kv_heads,
                    shape.head_dim, shape.intermediate, shape.vocab, int(shape.tie_embeddings),
                    shape.rms_eps, shape.rope_theta, 16, max_batch, max_pages_per_seq,
                    num_pages, int(use_graphs), int(persistent), int(max_prefill_rows),
                    int(bool(kv_fp8)), float(k_scale), float(v_scale))


def qd_create(cfg: QdConfig, stream: int = 0) -> int:
    lib = load_library()
    h = ctypes.c_void_p()
    rc = lib.qd_create(ctypes.byref(cfg), ctypes.c_void_p(stream), ctypes.byref(h))
    _check(rc, None)
    return h.value


def qd_load_weights(handle: int, tensors: Dict[str, object]) -> None:
    """tensors: HF name -> bf16 device tensor (torch.bfloat16 on the GPU)."""
    lib = load_library()
    descs = (QdTensorDesc * len(tensors))()
    keep = []
    for i, (name, t) in enumerate(tensors.items()):
        nb = name.encode()
        keep.append(nb)
        shape = tuple(t.shape)
        d = descs[i]
        d.name = nb
        d.data = _ptr(t)
        d.ndim = len(shape)
        d.shape[0] = shape[0]
        d.shape[1] = shape[1] if len(shape) > 1 else 0
        d.dtype = 0
    _check(lib.qd_load_weights(handle, descs, len(tensors)), handle)


def qd_decode_step(handle: int, batch: int, token_ids, positions, block_tables, kv_pool,
                   out_next_ids, out_logits=None) -> None:
    lib = load_library()
    _check(lib.qd_decode_step(handle, batch, _ptr(token_ids), _ptr(positions),
                              _ptr(block_tables), _ptr(kv_pool), _ptr(out_next_ids),
                              _ptr(out_logits)), handle)


def qd_prefill(handle: int, rows: int, token_ids, positions, block_tables, kv_pool,
               n_logits: int, out_next_ids=None, out_logits=None) -> None:
    lib = load_library()
    _check(lib.qd_prefill(handle, rows, _ptr(token_ids), _ptr(positions), _ptr(block_tables),
                          _ptr(kv_pool), n_logits, _ptr(out_next_ids), _ptr(out_logits)), handle)


def qd_prefill_prompts(handle: int, seq_rows, start_pos, token_ids, block_tables, kv_pool,
                       n_logits: int, out_next_ids=None, out_logits=None) -> None:
    """seq_rows, start_pos: host int sequences (one entry per prompt segment)."""
    lib = load_library()
    n = len(seq_rows)
    rows = np.ascontiguousarray(seq_rows, dtype=np.int32)
    pos = np.ascontiguousarray(start_pos, dtype=np.int32)
    if pos.shape != (n,):
        raise ValueError("seq_rows and start_pos differ in length")
    _check(lib.qd_prefill_prompts(handle, n, rows.ctypes.data, pos.ctypes.data, _ptr(token_ids),
                                  _ptr(block_tables), _ptr(kv_pool), n_logits,
                                  _ptr(out_next_ids), _ptr(out_logits)), handle)


def qd_decode_step_taps(handle: int, batch: int, token_ids, positions, block_tables, kv_pool,
                        out_next_ids, out_logits=None, taps: Optional[dict] = None,
                        tap_layer: int = -1) -> None:
    lib = load_library()
    tp = None
    if taps is not None:
        tp = QdTaps(tap_layer, *[_ptr(taps.get(n)) for n in TAP_NAMES])
    _check(lib.qd_decode_step_taps(handle, batch, _ptr(token_ids), _ptr(positions),
                                   _ptr(block_tables), _ptr(kv_pool), _ptr(out_next_ids),
                                   _ptr(out_logits), ctypes.byref(tp) if tp else None), handle)


def qd_stream_step_taps(handle: int, token_ids, positions, block_tables, kv_pool,
                        out_next_ids, out_logits=None, taps: Optional[dict] = None,
                        tap_layer: int = -1) -> None:
    lib = load_library()
    tp = None
    if taps is not None:
        tp = QdTaps(tap_layer, *[_ptr(taps.get(n)) for n in TAP_NAMES])
    _check(lib.qd_stream_step_taps(handle, _ptr(token_ids), _ptr(positions), _ptr(block_tables),
                                   _ptr(kv_pool), _ptr(out_next_ids), _ptr(out_logits),
                                   ctypes.byref(tp) if tp else None), handle)


def qd_sample_noalloc(batch: int, vocab: int, logits, temperature, top_k, top_p, uniform,
                      out_ids, stream: Optional[int] = None) -> None:
    """qd_sample without a handle; scratch is the library's static device array."""
    lib = load_library()
    _check(lib.qd_sample_noalloc(batch, vocab, _ptr(logits), _ptr(temperature), _ptr(top_k),
                                 _ptr(top_p), _ptr(uniform), _ptr(out_ids), stream), None)


def qd_read_ceiling(buf, nbytes: int, reps: int, stream: Optional[int] = None) -> float:
    """Plain streaming-read rate (GB/s) over the first nbytes of a device buffer."""
    lib = load_library()
    out = ctypes.c_float()
    _check(lib.qd_read_ceiling(_ptr(buf), int(nbytes), int(reps), stream, ctypes.byref(out)), None)
    return float(out.value)


def qd_profile_step(handle: int, batch: int, token_ids, positions, block_tables, kv_pool,
                    out_next_ids, out_logits=None):
    """One eager step timed per kernel class; returns {class: (ms, launches)}."""
    lib = load_library()
    n = len(PROF_CLASSES)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib.qd_profile_step(handle, batch, _ptr(token_ids), _ptr(positions),
                               _ptr(block_tables), _ptr(kv_pool), _ptr(out_next_ids),
                               _ptr(out_logits), ms, cnt), handle)
    return {PROF_CLASSES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


def qd_profile_class(handle: int, batch: int, cls: str, reps: int = 20) -> float:
    """Mean microseconds per launch of one projection class replayed alone."""
    lib = load_library()
    v = ctypes.c_float(0.0)
    _check(lib.qd_profile_class(handle, batch, PROF_CLASSES.index(cls), reps, ctypes.byref(v)),
           handle)
    return float(v.value)


def qd_sample(handle: int, batch: int, logits, temperature, top_k, top_p, uniform,
              out_ids) -> None:
    """Sampled next token per sequence from device logits [batch][vocab]; every
    argument is a device tensor of `batch` entries (see include/qd.h)."""
    lib = load_library()
    _check(lib.qd_sample(handle, batch, _ptr(logits), _ptr(temperature), _ptr(top_k),
                         _ptr(top_p), _ptr(uniform), _ptr(out_ids)), handle)


def qd_device_status(handle: int) -> int:
    lib = load_library()
    v = ctypes.c_int32(0)
    _check(lib.qd_device_status(handle, ctypes.byref(v)), handle)
    return v.value


def qd_stream(handle: int) -> int:
    return load_library().qd_stream(handle) or 0


STEP_PATHS = {0: "staged", 1: "graph", 3: "stream"}  # QD_PATH_* values


def qd_step_path(handle: int, batch: int) -> str:
    """How a step of `batch` sequences runs on this handle (see STEP_PATHS)."""
    v = load_library().qd_step_path(handle, batch)
    _check(v if v < 0 else 0, handle)
    return STEP_PATHS[v]


def qd_destroy(handle: int) -> None:
    load_library().qd_destroy(handle)


def qd_last_error(handle: Optional[int] = None) -> str:
    msg = load_library().qd_last_error(handle)
    return msg.decode() if msg else ""


class PageManager:
    """Host-side page manager of a paged KV pool (qd_blocks_* in include/qd.h).
    Methods return the C call's non-negative result and raise QdError on an
    error code (QD_ENOMEM: not enough pages, nothing changed)."""

    def __init__(self, num_pages: int, max_pages_per_seq: int):
        self.lib = load_library()
        h = ctypes.c_void_p()
        rc = self.lib.qd_blocks_create(num_pages, max_pages_per_seq, ctypes.byref(h))
        if rc != QD_OK:
            raise QdError(rc, "qd_blocks_create failed")
        self.h = h.value
        self.max_pages = max_pages_per_seq

    def _rc(self, rc: int) -> int:
        if rc < 0:
            raise QdError(rc, "page manager call failed")
        return rc

    def add(self, seq: int) -> None:
        self._rc(self.lib.qd_blocks_add(self.h, seq))

    def reserve(self, seq: int, n_tokens: int) -> None:
        self._rc(self.lib.qd_blocks_reserve(self.h, seq, n_tokens))

    def release(self, seq: int) -> None:
        self._rc(self.lib.qd_blocks_release(self.h, seq))

    def fork(self, src: int, dst: int):
        """(copy_src, copy_dst): the page to copy on the device, or (-1, -1)."""
        a, b = ctypes.c_int32(), ctypes.c_int32()
        self._rc(self.lib.qd_blocks_fork(self.h, src, dst, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def tables(self, seqs, pad_page: int) -> np.ndarray:
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        out = np.empty((len(ids), self.max_pages), dtype=np.int32)
        self._rc(self.lib.qd_blocks_tables(self.h, ids.ctypes.data, len(ids), pad_page,
                                           out.ctypes.data))
        return out

    def length(self, seq: int) -> int:
        return self._rc(self.lib.qd_blocks_length(self.h, seq))

    def available(self) -> int:
        return self._rc(self.lib.qd_blocks_available(self.h))

    def publish(self, seq: int, tokens) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        return self._rc(self.lib.qd_blocks_publish(self.h, seq, t.ctypes.data, len(t)))

    def match(self, seq: int, tokens) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        return self._rc(self.lib.qd_blocks_match(self.h, seq, t.ctypes.data, len(t)))

    def close(self) -> None:
        if self.h:
            self.lib.qd_blocks_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Engine:
    """Continuous-batching serving loop over a handle and its KV pool
    (qd_engine_* in include/qd.h).  submit() queues a request; step() runs
    one iteration and returns [(request id, token, finished)]."""

    def __init__(self, handle: int, kv_pool, max_batch: int):
        self.lib = load_library()
        self.handle = handle
        self.max_out = max_batch
        e = ctypes.c_void_p()
        _check(self.lib.qd_engine_create(handle, _ptr(kv_pool), ctypes.byref(e)), handle)
        self.e = e.value
        self._req = np.empty(max_batch, dtype=np.int64)
        self._tok = np.empty(max_batch, dtype=np.int32)
        self._done = np.empty(max_batch, dtype=np.int32)

    def submit(self, req: int, prompt, max_new_tokens: int, eos_id: int = -1,
               temperature: float = 0.0, top_k: int = 0, top_p: float = 1.0,
               seed: int = 0) -> None:
        """Queue a request (greedy when temperature <= 0; see qd_engine_request)."""
        t = np.ascontiguousarray(prompt, dtype=np.int32)
        r = QdEngineRequest(req, t.ctypes.data if len(t) else None, len(t), max_new_tokens, eos_id,
                            temperature, top_k, top_p, seed & (2 ** 64 - 1))
        _check(self.lib.qd_engine_submit(self.e, ctypes.byref(r)), self.handle)

    def step(self):
        n = ctypes.c_int32()
        _check(self.lib.qd_engine_step(self.e, self.max_out, self._req.ctypes.data,
                                       self._tok.ctypes.data, self._done.ctypes.data,
                                       ctypes.byref(n)), self.handle)
        return [(int(self._req[i]), int(self._tok[i]), bool(self._done[i])) for i in range(n.value)]

    def stats(self) -> dict:
        st = QdEngineStats()
        _check(self.lib.qd_engine_get_stats(self.e, ctypes.byref(st)), self.handle)
        return {name: getattr(st, name) for name, _ in QdEngineStats._fields_ if name != "reserved"}

    def close(self) -> None:
        if self.e:
            self.lib.qd_engine_destroy(self.e)
            self.e = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
