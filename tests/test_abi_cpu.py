"""CPU-only checks of the C ABI: the library loads, exports every function
include/moe.h declares, and rejects bad arguments on the host before any
HIP call (so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def q():
    import quantized_moe_route_amd as q
    return q


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(q):
    names = _declared()
    assert {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine"} <= set(names)
    lib = C.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q.ENTRY_POINTS)


def test_version_and_status_strings(q):
    assert q.moe_abi_version() == 1
    for s in range(5):
        assert isinstance(q.moe_status_string(s), str) and q.moe_status_string(s)


A = 4096  # a 256-aligned fake device address; validation fails before it is used


def test_route_validation(q):
    E_ = q.MOE_ERR_INVALID_ARGUMENT
    r = lambda *a: q.moe_route(*a, check=False)
    assert r(A, A, None, A, 1, 2048, 0, 1, A, A, A, 1 << 20) == E_          # E < 1
    assert r(A, A, None, A, 1, 2048, 1025, 1, A, A, A, 1 << 20) == E_       # E > 1024
    assert r(A, A, None, A, 1, 2048, 16, 17, A, A, A, 1 << 20) == E_        # k > E
    assert r(A, A, None, A, -1, 2048, 16, 2, A, A, A, 1 << 20) == E_        # T < 0
    assert r(None, A, None, A, 1, 2048, 16, 2, A, A, A, 1 << 20) == E_      # x missing
    assert r(A, None, A, A, 1, 2048, 16, 2, A, A, A, 1 << 20) == E_         # logits-in with bias
    assert r(A + 4, A, None, A, 1, 2048, 16, 2, A, A, A, 1 << 20) == E_     # misaligned
    assert r(A, A, None, A, 1, 2000, 16, 2, A, A, A, 1 << 20) == q.MOE_ERR_UNSUPPORTED
    assert r(A, A, None, A, 1, 2048, 16, 2, A, A, None, 0) == q.MOE_ERR_WORKSPACE
    assert r(A, A, None, A, 1, 2048, 16, 2, A, A, A + 16, 1 << 20) == q.MOE_ERR_WORKSPACE
    assert r(A, A, None, A, 4, 2048, 512, 10, A, A, A, 4096) == q.MOE_ERR_WORKSPACE
    assert r(A, A, None, A, 0, 2048, 16, 2, A, A, A, 1 << 20) == q.MOE_OK    # T = 0: no-op


def test_dispatch_and_combine_validation(q):
    d = lambda *a: q.moe_dispatch(*a, check=False)
    assert d(None, 4, 16, 2, A, A, A, A, 1 << 20) == q.MOE_ERR_INVALID_ARGUMENT
    assert d(A, 4, 16, 0, A, A, A, A, 1 << 20) == q.MOE_ERR_INVALID_ARGUMENT
    assert d(A, 4, 16, 2, A, A, A, None, 0) == q.MOE_ERR_WORKSPACE
    assert d(A, 0, 16, 2, A, A, A, A, 1 << 20) == q.MOE_OK
    ts = lambda *a: q.moe_dispatch_tail_skip(*a, check=False)
    assert ts(A, 4, 16, 2, -1, A, A, A, A, 1 << 20) == q.MOE_ERR_INVALID_ARGUMENT   # tail_from < 0
    assert ts(A, 4, 16, 2, 3, A, A, A, A, 1 << 20) == q.MOE_ERR_INVALID_ARGUMENT    # tail_from > k
    assert ts(None, 4, 16, 2, 1, A, A, A, A, 1 << 20) == q.MOE_ERR_INVALID_ARGUMENT
    assert ts(A, 4, 16, 2, 1, A, A, A, None, 0) == q.MOE_ERR_WORKSPACE
    assert ts(A, 0, 16, 2, 2, A, A, A, A, 1 << 20) == q.MOE_OK
    rd = lambda *a: q.moe_route_dispatch(*a, check=False)
    assert rd(A, None, None, A, 1, 2048, 16, 2, A, A, A, A, A, A, 1 << 24) == q.MOE_ERR_INVALID_ARGUMENT
    assert rd(A, A, None, A, 1, 2048, 16, 2, A, A, None, A, A, A, 1 << 24) == q.MOE_ERR_INVALID_ARGUMENT
    assert rd(A, A, None, A, 1, 100, 16, 2, A, A, A, A, A, A, 1 << 24) == q.MOE_ERR_UNSUPPORTED
    assert rd(A, A, None, A, 1, 2048, 16, 2, A, A, A, A, A, A, 4096) == q.MOE_ERR_WORKSPACE
    assert rd(A, A, None, A, 0, 2048, 16, 2, A, A, A, A, A, A, 1 << 24) == q.MOE_OK
    c = lambda *a: q.moe_combine(*a, check=False)
    assert c(A, A, A, A, 3, 2, 2048, None) == q.MOE_ERR_INVALID_ARGUMENT
    assert c(A, A, A, A, 3, 2, 100, A) == q.MOE_ERR_UNSUPPORTED
    assert c(A, A, A, A, 3, 0, 2048, A) == q.MOE_ERR_INVALID_ARGUMENT
    assert c(A, A, A, A, 0, 2, 2048, A) == q.MOE_OK


def _layer(q, fmt=1, d=256, f=128, E=16, hi=None, mn=A):
    qm = q.make_qmat(A, hi, A, mn)
    return q.moe_layer(fmt, d, f, E, qm, qm, qm, qm, qm, qm)


def test_ffn_validation(q):
    f = lambda L, *a: q.moe_expert_ffn(L, *a, check=False)
    ws = 1 << 24
    assert f(_layer(q, fmt=3), A, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_UNSUPPORTED
    assert f(_layer(q, d=200), A, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_UNSUPPORTED
    assert f(_layer(q, hi=A), A, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT  # Q2 with hi
    assert f(_layer(q, fmt=2, hi=None, mn=None), A, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q, fmt=2, hi=A, mn=A), A, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), None, 4, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 17, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, A, A, A, A, A, 16) == q.MOE_ERR_WORKSPACE
    assert f(_layer(q), A, 0, 2, A, A, A, A, A, ws) == q.MOE_OK


def test_routed_and_shared_ffn_validation(q):
    r = lambda L, *a: q.moe_routed_ffn(L, *a, check=False)
    s = lambda L, *a: q.moe_shared_ffn(L, *a, check=False)
    ws = 1 << 24
    good, none = q.make_qmat(A, None, A, A), q.make_qmat(None, None, None, None)
    routed_only = q.moe_layer(1, 256, 128, 16, good, good, good, none, none, none)
    shared_only = q.moe_layer(1, 256, 128, 16, none, none, none, good, good, good)
    # moe_routed_ffn(layer, x, T, k, offsets, sorted_pair, y_pairs, ws, ws_bytes)
    assert r(_layer(q), A, 4, 2, None, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert r(_layer(q), A, 4, 2, A, None, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert r(_layer(q), A, 4, 2, A, A, None, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert r(_layer(q), A, 4, 0, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert r(_layer(q), A, 4, 2, A, A, A, A, 16) == q.MOE_ERR_WORKSPACE
    assert r(shared_only, A, 4, 2, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert r(routed_only, A, 0, 2, A, A, A, A, ws) == q.MOE_OK   # shared matrices not needed
    # moe_shared_ffn(layer, x, T, y_shared, ws, ws_bytes)
    assert s(_layer(q), None, 4, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert s(_layer(q), A, 4, None, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert s(_layer(q), A, -1, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert s(_layer(q), A, 4, A, A, 16) == q.MOE_ERR_WORKSPACE
    assert s(routed_only, A, 4, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert s(shared_only, A, 0, A, A, ws) == q.MOE_OK            # routed matrices not needed
    # moe_expert_ffn needs both
    f = lambda L, *a: q.moe_expert_ffn(L, *a, check=False)
    assert f(routed_only, A, 0, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(shared_only, A, 0, 2, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT


def test_route_dispatch_tail_skip_validation(q):
    rd = lambda *a: q.moe_route_dispatch_tail_skip(*a, check=False)
    # (x, wr, bias, logits, T, d, E, k, tail_from, ids, w, offsets, sorted_pair, pair_pos, ws, ws_bytes)
    assert rd(A, A, None, A, 1, 2048, 16, 2, 3, A, A, A, A, A, A, 1 << 24) == q.MOE_ERR_INVALID_ARGUMENT
    assert rd(A, A, None, A, 1, 2048, 16, 2, -1, A, A, A, A, A, A, 1 << 24) == q.MOE_ERR_INVALID_ARGUMENT
    assert rd(A, A, None, A, 1, 2048, 16, 2, 1, A, A, A, A, A, A, 4096) == q.MOE_ERR_WORKSPACE
    assert rd(A, A, None, A, 0, 2048, 16, 2, 1, A, A, A, A, A, A, 1 << 24) == q.MOE_OK


def test_ffn_combine_validation(q):
    f = lambda L, *a: q.moe_expert_ffn_combine(L, *a, check=False)
    ws = 1 << 24
    # (x, T, k, offsets, sorted_pair, pair_pos, topk_w, y_pairs, y_shared, out, ws, ws_bytes)
    assert f(_layer(q), A, 4, 2, A, A, None, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, A, A, A, None, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, A, A, A, A, A, A, None, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, None, A, A, A, A, A, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, A, A, A, A, A, None, A, A, ws) == q.MOE_ERR_INVALID_ARGUMENT
    assert f(_layer(q), A, 4, 2, A, A, A, A, A, A, A, A, 16) == q.MOE_ERR_WORKSPACE
    assert f(_layer(q), A, 40, 2, A, A, A, A, A, A, A, A, 16) == q.MOE_ERR_WORKSPACE
    assert f(_layer(q, fmt=3), A, 4, 2, A, A, A, A, A, A, A, A, ws) == q.MOE_ERR_UNSUPPORTED
    assert f(_layer(q), A, 0, 2, A, A, A, A, A, A, A, A, ws) == q.MOE_OK


def test_workspace_size_monotone(q):
    s1 = q.moe_workspace_size(2048, 768, 512, 1, 10)
    s4 = q.moe_workspace_size(2048, 768, 512, 4, 10)
    s8k = q.moe_workspace_size(2048, 768, 512, 8192, 10)
    assert 0 < s1 <= s4 <= s8k and s1 % 256 == 0


def test_validate_ids_host(q):
    """moe_validate_ids: the preconditions moe_dispatch states on its ids
    (range [0, E), distinct within a token), checked on a host array."""
    import numpy as np
    v = lambda ids, T, E, k: q.moe_validate_ids(ids, T, E, k, check=False)
    ok = np.array([[3, 1], [0, 15], [15, 14]], np.int32)
    assert v(ok, 3, 16, 2) == q.MOE_OK
    assert v(np.array([[3, 16]], np.int32), 1, 16, 2) == q.MOE_ERR_INVALID_ARGUMENT     # id = E
    assert v(np.array([[-1, 2]], np.int32), 1, 16, 2) == q.MOE_ERR_INVALID_ARGUMENT     # negative id
    assert v(np.array([[5, 5]], np.int32), 1, 16, 2) == q.MOE_ERR_INVALID_ARGUMENT      # repeated
    # the same expert in different tokens is fine
    assert v(np.array([[5, 6], [6, 5]], np.int32), 2, 16, 2) == q.MOE_OK
    assert v(None, 0, 16, 2) == q.MOE_OK                                                # T = 0
    assert v(None, 2, 16, 2) == q.MOE_ERR_INVALID_ARGUMENT
    assert v(ok, 3, 16, 17) == q.MOE_ERR_INVALID_ARGUMENT                                # k > E
    assert v(ok, 3, 1025, 2) == q.MOE_ERR_INVALID_ARGUMENT                               # E > 1024
    # every generated routing of the workloads' shapes passes; k = E is a permutation
    rng = np.random.default_rng(3)
    for E, k, T in ((512, 10, 64), (16, 16, 5), (1024, 1024, 2), (1, 1, 7)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        assert v(ids, T, E, k) == q.MOE_OK
        bad = ids.copy()
        bad[T - 1, k - 1] = E
        assert v(bad, T, E, k) == q.MOE_ERR_INVALID_ARGUMENT


def test_error_word_layout_matches_header(q):
    """The error word sits inside the router's 4 KiB counter block, past the
    token-tile counters (16 tiles x 128 bytes), and the binding agrees with
    the header."""
    src = open(HEADER).read()
    off = int(re.search(r"#define MOE_WS_ERROR_OFFSET (\d+)", src).group(1))
    assert off == q.MOE_WS_ERROR_OFFSET
    assert 2048 <= off and off + 4 <= 4096 and off % 4 == 0
    assert int(re.search(r"#define MOE_WS_ERR_ID_RANGE (\d+)", src).group(1)) == q.MOE_WS_ERR_ID_RANGE
    assert int(re.search(r"#define MOE_WS_ERR_ID_REPEAT (\d+)", src).group(1)) == q.MOE_WS_ERR_ID_REPEAT
