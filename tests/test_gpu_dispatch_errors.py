"""GPU: moe_dispatch on ids that break its preconditions.

The dispatch kernels range-check every id before it indexes anything (the
kernels' own bounds checks; no access leaves its buffer): a pair whose id
lies outside [0, E) is left out of the listing and sets MOE_WS_ERR_ID_RANGE
in the workspace's error word; a token naming one expert twice sets
MOE_WS_ERR_ID_REPEAT.  Both dispatch paths (one block for small batches,
count/scan/place for large ones), with and without route tail-skip.
Valid ids leave the error word at zero.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_route_amd as q
    return q


def _ws(q, E, T, k):
    nbytes = q.moe_workspace_size(256, 128, E, T, k)
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-t.data_ptr()) % 256
    ws = t[off:off + nbytes]
    q.moe_workspace_init(ws, nbytes)
    return ws, nbytes


def _err_word(q, ws):
    o = q.MOE_WS_ERROR_OFFSET
    return int(ws[o:o + 4].cpu().numpy().view(np.int32)[0])


def _dispatch(q, ids, E, tail_from=None):
    T, k = ids.shape
    P = T * k
    ws, nbytes = _ws(q, E, T, k)
    dev = torch.from_numpy(ids).cuda()
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    pp = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    if tail_from is None:
        q.moe_dispatch(dev, T, E, k, off, sp, pp, ws, nbytes)
    else:
        q.moe_dispatch_tail_skip(dev, T, E, k, tail_from, off, sp, pp, ws, nbytes)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), pp.cpu().numpy(), _err_word(q, ws)


def _routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


# (T, E, k): one-block path and count/scan/place path
SHAPES = [(4, 16, 2), (37, 64, 8), (1000, 512, 10)]


@pytest.mark.parametrize("T,E,k", SHAPES)
@pytest.mark.parametrize("tail_from", [None, 1])
def test_out_of_range_ids_are_dropped_and_flagged(q, T, E, k, tail_from):
    rng = np.random.default_rng(T + E)
    ids = _routing(rng, T, E, k)
    bad = rng.choice(T * k, size=max(1, T * k // 50), replace=False)
    vals = np.array([E, -1, E + 1000, np.iinfo(np.int32).max, np.iinfo(np.int32).min], np.int32)
    ids.reshape(-1)[bad] = vals[np.arange(len(bad)) % len(vals)]
    print(f"T={T} E={E} k={k} tail_from={tail_from}: {len(bad)} bad ids", flush=True)
    off, sp, pp, err = _dispatch(q, ids, E, tail_from)
    assert err & q.MOE_WS_ERR_ID_RANGE
    assert not err & q.MOE_WS_ERR_ID_REPEAT
    # expected: the listing of the valid pairs alone (bad pairs behave as dropped)
    valid = (ids >= 0) & (ids < E)
    masked = np.where(valid, ids, 0)
    if tail_from is None:
        keep_e = np.ones(E, bool)
    else:
        keep_e = np.zeros(E, bool)
        for t in range(T):
            for j in range(min(tail_from, k)):
                if valid[t, j]:
                    keep_e[ids[t, j]] = True
    listed = valid & keep_e[masked]
    flat_e, flat_ok = masked.ravel(), listed.ravel()
    order = [p for e in range(E) for p in range(T * k) if flat_ok[p] and flat_e[p] == e]
    n = len(order)
    assert off[E] == n
    assert np.array_equal(sp[:n], np.array(order, np.int32))
    pos_ref = np.full(T * k, -1, np.int32)
    pos_ref[np.array(order, dtype=np.int64)] = np.arange(n, dtype=np.int32)
    assert np.array_equal(pp, pos_ref)
    counts = np.bincount(flat_e[flat_ok], minlength=E)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_repeated_ids_are_flagged_and_listing_stays_valid(q, T, E, k):
    rng = np.random.default_rng(7 * T + E)
    ids = _routing(rng, T, E, k)
    rows = rng.choice(T, size=max(1, T // 10), replace=False)
    ids[rows, k - 1] = ids[rows, 0]
    off, sp, pp, err = _dispatch(q, ids, E)
    assert err & q.MOE_WS_ERR_ID_REPEAT
    n = off[E]
    assert 0 <= n <= T * k and np.all(np.diff(off) >= 0) and off[0] == 0
    assert np.all((sp[:n] >= 0) & (sp[:n] < T * k))
    assert np.all((pp >= 0) & (pp < n))
    # each listed entry is a pair of the expert whose segment holds it
    seg = np.searchsorted(off, np.arange(n), side="right") - 1
    assert np.array_equal(ids.ravel()[sp[:n]], seg)


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_valid_ids_leave_error_word_zero(q, T, E, k):
    ids = _routing(np.random.default_rng(11), T, E, k)
    off, sp, pp, err = _dispatch(q, ids, E)
    assert err == 0
    off_ref, sp_ref, pp_ref = oracle.dispatch(ids, E)
    assert np.array_equal(off, off_ref) and np.array_equal(sp, sp_ref) and np.array_equal(pp, pp_ref)
