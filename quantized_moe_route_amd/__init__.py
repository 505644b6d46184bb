"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every computation runs in the HIP kernels of libmoe.so; PyTorch provides
device memory and streams.  The functions below have the same names and
arguments as the C entry points (device tensors stand in for pointers, a
torch stream or None for the hipStream_t) and raise MoeError on a non-OK
status.  Importing this module loads the in-tree library and fails loudly
if it has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_FMT_Q2_B32, MOE_FMT_Q3_B32 = 1, 2
ENTRY_POINTS = ("moe_route", "moe_dispatch", "moe_dispatch_tail_skip", "moe_route_dispatch",
                "moe_route_dispatch_tail_skip",
                "moe_expert_ffn", "moe_routed_ffn", "moe_shared_ffn", "moe_expert_ffn_combine",
                "moe_expert_ffn_noalloc",
                "moe_combine", "moe_validate_ids", "moe_workspace_size", "moe_workspace_init",
                "moe_status_string", "moe_abi_version")
MOE_WS_ERROR_OFFSET = 3968                          # byte offset of the workspace's error word
MOE_WS_ERR_ID_RANGE, MOE_WS_ERR_ID_REPEAT = 1, 2    # its bits


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


class moe_qmat(C.Structure):
    _fields_ = [("lo", C.c_void_p), ("hi", C.c_void_p), ("scale", C.c_void_p), ("min", C.c_void_p)]


class moe_layer(C.Structure):
    _fields_ = [("format", C.c_int32), ("d_model", C.c_int32), ("d_ff", C.c_int32),
                ("n_experts", C.c_int32), ("gate", moe_qmat), ("up", moe_qmat), ("down", moe_qmat),
                ("sh_gate", moe_qmat), ("sh_up", moe_qmat), ("sh_down", moe_qmat)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoe.so not built ({LIB_PATH}); run __graft_entry__.build() or "
                          "python quantized_moe_route_amd/_build.py")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    lib.moe_route.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.moe_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_dispatch_tail_skip.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_route_dispatch.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_dispatch_tail_skip.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                 vp, sz, vp]
    lib.moe_expert_ffn.argtypes = [C.POINTER(moe_layer), vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_routed_ffn.argtypes = [C.POINTER(moe_layer), vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_shared_ffn.argtypes = [C.POINTER(moe_layer), vp, i32, vp, vp, sz, vp]
    lib.moe_expert_ffn_combine.argtypes = [C.POINTER(moe_layer), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                           vp, sz, vp]
    lib.moe_expert_ffn_noalloc.argtypes = [C.POINTER(moe_layer), vp, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.moe_validate_ids.argtypes = [vp, i32, i32, i32]
    lib.moe_validate_ids.restype = C.c_int
    lib.moe_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.moe_workspace_size.restype = sz
    lib.moe_workspace_init.argtypes = [vp, sz, vp]
    lib.moe_status_string.argtypes = [C.c_int]
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_abi_version.restype = i32
    for f in ("moe_route", "moe_dispatch", "moe_dispatch_tail_skip", "moe_route_dispatch", "moe_expert_ffn",
              "moe_expert_ffn_noalloc", "moe_combine", "moe_workspace_init"):
        getattr(lib, f).restype = C.c_int
    return lib


lib = _load()


def _ptr(t):
    """Device tensor (or raw int address, or None) -> address."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int, call: str) -> int:
    if st != MOE_OK:
        raise MoeError(st, call)
    return st


def status_string(st: int) -> str:
    return lib.moe_status_string(st).decode()


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_string(st: int) -> str:
    return status_string(st)


def moe_validate_ids(topk_ids_host, T, E, k, check=True):
    """topk_ids_host: a HOST int32 array [T][k] (numpy), checked on the host."""
    import numpy as np
    a = None if topk_ids_host is None else np.ascontiguousarray(topk_ids_host, dtype=np.int32)
    st = lib.moe_validate_ids(None if a is None else a.ctypes.data, T, E, k)
    return _check(st, "moe_validate_ids") if check else st


def moe_workspace_size(d_model, d_ff, E, T, k) -> int:
    return lib.moe_workspace_size(d_model, d_ff, E, T, k)


def moe_workspace_init(ws, ws_bytes, stream=None):
    return _check(lib.moe_workspace_init(_ptr(ws), ws_bytes, _stream(stream)), "moe_workspace_init")


def moe_route(x_bf16, w_router, bias, logits, T, d_model, E, k, topk_ids, topk_w, ws, ws_bytes,
              stream=None, check=True):
    st = lib.moe_route(_ptr(x_bf16), _ptr(w_router), _ptr(bias), _ptr(logits), T, d_model, E, k,
                       _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_route") if check else st


def moe_dispatch(topk_ids, T, E, k, offsets, sorted_pair, pair_pos, ws, ws_bytes, stream=None,
                 check=True):
    st = lib.moe_dispatch(_ptr(topk_ids), T, E, k, _ptr(offsets), _ptr(sorted_pair),
                          _ptr(pair_pos), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_dispatch") if check else st


def moe_dispatch_tail_skip(topk_ids, T, E, k, tail_from, offsets, sorted_pair, pair_pos, ws, ws_bytes,
                           stream=None, check=True):
    st = lib.moe_dispatch_tail_skip(_ptr(topk_ids), T, E, k, tail_from, _ptr(offsets), _ptr(sorted_pair),
                                    _ptr(pair_pos), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_dispatch_tail_skip") if check else st


def moe_route_dispatch(x_bf16, w_router, bias, logits, T, d_model, E, k, topk_ids, topk_w, offsets,
                       sorted_pair, pair_pos, ws, ws_bytes, stream=None, check=True):
    st = lib.moe_route_dispatch(_ptr(x_bf16), _ptr(w_router), _ptr(bias), _ptr(logits), T, d_model, E, k,
                                _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(sorted_pair),
                                _ptr(pair_pos), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_route_dispatch") if check else st

def moe_route_dispatch_tail_skip(x_bf16, w_router, bias, logits, T, d_model, E, k, tail_from, topk_ids,
                                 topk_w, offsets, sorted_pair, pair_pos, ws, ws_bytes, stream=None,
                                 check=True):
    st = lib.moe_route_dispatch_tail_skip(_ptr(x_bf16), _ptr(w_router), _ptr(bias), _ptr(logits), T, d_model,
                                          E, k, tail_from, _ptr(topk_ids), _ptr(topk_w), _ptr(offsets),
                                          _ptr(sorted_pair), _ptr(pair_pos), _ptr(ws), ws_bytes,
                                          _stream(stream))
    return _check(st, "moe_route_dispatch_tail_skip") if check else st


def moe_expert_ffn(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, ws, ws_bytes,
                   stream=None, check=True):
    st = lib.moe_expert_ffn(C.byref(layer), _ptr(x_bf16), T, k, _ptr(offsets), _ptr(sorted_pair),
                            _ptr(y_pairs), _ptr(y_shared), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_expert_ffn") if check else st


def moe_expert_ffn_noalloc(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, stream=None,
                           check=True):
    st = lib.moe_expert_ffn_noalloc(C.byref(layer), _ptr(x_bf16), T, k, _ptr(offsets), _ptr(sorted_pair),
                                    _ptr(y_pairs), _ptr(y_shared), _stream(stream))
    return _check(st, "moe_expert_ffn_noalloc") if check else st


def moe_routed_ffn(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, ws, ws_bytes, stream=None,
                   check=True):
    st = lib.moe_routed_ffn(C.byref(layer), _ptr(x_bf16), T, k, _ptr(offsets), _ptr(sorted_pair),
                            _ptr(y_pairs), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_routed_ffn") if check else st


def moe_shared_ffn(layer, x_bf16, T, y_shared, ws, ws_bytes, stream=None, check=True):
    st = lib.moe_shared_ffn(C.byref(layer), _ptr(x_bf16), T, _ptr(y_shared), _ptr(ws), ws_bytes,
                            _stream(stream))
    return _check(st, "moe_shared_ffn") if check else st


def moe_expert_ffn_combine(layer, x_bf16, T, k, offsets, sorted_pair, pair_pos, topk_w, y_pairs,
                           y_shared, out, ws, ws_bytes, stream=None, check=True):
    st = lib.moe_expert_ffn_combine(C.byref(layer), _ptr(x_bf16), T, k, _ptr(offsets),
                                    _ptr(sorted_pair), _ptr(pair_pos), _ptr(topk_w), _ptr(y_pairs),
                                    _ptr(y_shared), _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    return _check(st, "moe_expert_ffn_combine") if check else st


def moe_combine(y_pairs, y_shared, pair_pos, topk_w, T, k, d_model, out, stream=None, check=True):
    st = lib.moe_combine(_ptr(y_pairs), _ptr(y_shared), _ptr(pair_pos), _ptr(topk_w), T, k,
                         d_model, _ptr(out), _stream(stream))
    return _check(st, "moe_combine") if check else st


def make_qmat(lo, hi, scale, mn) -> moe_qmat:
    return moe_qmat(_ptr(lo), _ptr(hi), _ptr(scale), _ptr(mn))


def make_layer(fmt, d_model, d_ff, n_experts, mats: dict) -> moe_layer:
    """mats: name -> (lo, hi, scale, min) device tensors for gate, up, down,
    sh_gate, sh_up, sh_down."""
    q = {n: make_qmat(*mats[n]) for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")}
    return moe_layer(fmt, d_model, d_ff, n_experts, q["gate"], q["up"], q["down"], q["sh_gate"],
                     q["sh_up"], q["sh_down"])
