"""Python access to the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg; the GPU library never imports, links or calls it.

`build()` compiles the C file with gcc (OpenMP, -O2); the functions below
marshal numpy arrays into it.  Matrices are passed as any object with the
attributes lo, hi, scale, min (numpy arrays, hi/min may be None), e.g. the
host copies made by the shared synthetic-input generator.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

Q2, Q3 = 1, 2


def build() -> str:
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"],
                   check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _QMat(C.Structure):
    _fields_ = [("lo", C.c_void_p), ("hi", C.c_void_p), ("scale", C.c_void_p), ("min", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(_LIB)
        _lib.oracle_bf16_to_double.restype = C.c_double
        _lib.oracle_fp16_to_double.restype = C.c_double
        _lib.oracle_weight.restype = C.c_double
        _lib.oracle_num_threads.restype = C.c_int
    return _lib


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _qm(m):
    """Keep references alive: returns (struct, arrays)."""
    arrs = [None if a is None else np.ascontiguousarray(a) for a in (m.lo, m.hi, m.scale, m.min)]
    return _QMat(*[None if a is None else a.ctypes.data for a in arrs]), arrs


def num_threads() -> int:
    return lib().oracle_num_threads()


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(C.c_uint16(b))


def fp16_to_double(b: int) -> float:
    return lib().oracle_fp16_to_double(C.c_uint16(b))


def code(m, fmt, rows, K, e, r, k) -> int:
    s, keep = _qm(m)
    return lib().oracle_code(C.byref(s), fmt, rows, K, e, r, k)


def weight(m, fmt, rows, K, e, r, k) -> float:
    s, keep = _qm(m)
    return lib().oracle_weight(C.byref(s), fmt, rows, K, e, r, k)


def dequant_matrix(m, fmt, rows, K, e=0) -> np.ndarray:
    s, keep = _qm(m)
    out = np.empty((rows, K), np.float64)
    lib().oracle_dequant_matrix(C.byref(s), fmt, rows, K, e, _p(out))
    return out


def router_logits(x_bits, wr, bias=None) -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    wr = np.ascontiguousarray(wr, np.float32)
    T, d = x_bits.shape
    E = wr.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_p(x_bits), _p(wr), _p(b), T, d, E, _p(out))
    return out


def topk_softmax(logits, k):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().oracle_topk_softmax(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def dispatch(ids, E):
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    lib().oracle_dispatch(_p(ids), T, k, E, _p(offsets), _p(sp), _p(pp))
    return offsets, sp, pp


def dispatch_tail_skip(ids, E, tail_from):
    """dispatch() without the pairs of experts that every token of the batch
    picked only at rank >= tail_from (0-based); those pairs get pair_pos -1."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    lib().oracle_dispatch_tail_skip(_p(ids), T, k, E, int(tail_from), _p(offsets), _p(sp), _p(pp))
    return offsets, sp, pp


def tail_keep(ids, E, tail_from):
    """keep[e]: expert e is picked at some rank < tail_from in the batch."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    keep = np.empty(E, np.int8)
    lib().oracle_tail_keep(_p(ids), T, k, E, int(tail_from), _p(keep))
    return keep.astype(bool)


def _layer_structs(L):
    parts = [_qm(getattr(L, n)) for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")]
    return [C.byref(p[0]) for p in parts], parts


def expert_rows(L, fmt, d, f, E, x_bits, row_expert, row_token, want_h=False, f64=False):
    """y[r] (and h[r]) for rows (row_expert[r], row_token[r]); expert -1 = shared."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    re = np.ascontiguousarray(row_expert, np.int32)
    rt = np.ascontiguousarray(row_token, np.int32)
    n = re.shape[0]
    dt = np.float64 if f64 else np.float32
    y = np.empty((n, d), dt)
    h = np.empty((n, f), dt) if want_h else None
    refs, keep = _layer_structs(L)
    fn = lib().oracle_expert_rows_f64 if f64 else lib().oracle_expert_rows
    fn(*refs, fmt, d, f, E, _p(x_bits), n, _p(re), _p(rt), _p(y), _p(h))
    return (y, h) if want_h else y


def combine(y_pairs, y_shared, pair_pos, w, T, k, d) -> np.ndarray:
    y_pairs = np.ascontiguousarray(y_pairs, np.float32)
    y_shared = np.ascontiguousarray(y_shared, np.float32)
    pair_pos = np.ascontiguousarray(pair_pos, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    out = np.empty((T, d), np.float32)
    lib().oracle_combine(_p(y_pairs), _p(y_shared), _p(pair_pos), _p(w), T, k, d, _p(out))
    return out


def layer(L, fmt, d, f, E, k, x_bits, wr=None, bias=None, logits=None, tail_from=None):
    """Whole layer; returns (ids, w, out).  Give `logits` to route on fixed logits;
    `tail_from` < k skips the experts the batch picked only at ranks >= tail_from."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    T = x_bits.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    out = np.empty((T, d), np.float32)
    wr = None if wr is None else np.ascontiguousarray(wr, np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lg = None if logits is None else np.ascontiguousarray(logits, np.float32)
    refs, keep = _layer_structs(L)
    tf = k if tail_from is None else int(tail_from)
    lib().oracle_layer(*refs, fmt, d, f, E, k, T, _p(x_bits), _p(wr), _p(b), _p(lg), tf,
                       _p(ids), _p(w), _p(out))
    return ids, w, out
