"""GPU parity, route tail-skip (moe_dispatch_tail_skip): the permutation is
bit-exact against the oracle's tail-skip dispatch, and the layer output with
the skip matches the oracle's layer with the same rank threshold
(max|gpu - oracle| <= 2e-3 * rms(oracle out)).  The rule: an expert that every
token of the batch picked only at ranks >= tail_from is not computed (the
page's case: ranks 7..10 of a top-10, tail_from = 6).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_route_amd as q
    return q


def _rel_err(gpu, ref):
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / rms)


@pytest.mark.parametrize("T,E,k,tail_from,skew", [
    (1, 512, 10, 6, 0.0), (4, 512, 10, 6, 1.1), (16, 64, 8, 3, 0.0), (65, 16, 16, 5, 0.0),
    (300, 1024, 16, 16, 0.0), (8192, 512, 10, 6, 1.3), (1000, 64, 8, 0, 0.0), (2048, 512, 10, 1, 0.0),
])
def test_dispatch_tail_skip_parity(q, T, E, k, tail_from, skew):
    """Small (one block) and large (count/scan/place) dispatch paths, with the
    keep rule, tail_from = k (no skip) and tail_from = 0 (all dropped)."""
    print(f"T={T} E={E} k={k} tail_from={tail_from}", flush=True)
    rng = np.random.default_rng(T * 7 + E + k + tail_from)
    if skew > 0:   # Zipf-like preference: low expert ids are picked more often
        pref = 1.0 / np.arange(1, E + 1) ** skew
        ids = np.stack([rng.choice(E, size=k, replace=False, p=pref / pref.sum()) for _ in range(T)])
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    ids = ids.astype(np.int32)
    ws_bytes = q.moe_workspace_size(128, 128, E, T, k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    ids_d = torch.from_numpy(ids).cuda()
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    pp = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    q.moe_dispatch_tail_skip(ids_d, T, E, k, tail_from, off, sp, pp, ws, ws_bytes)
    torch.cuda.synchronize()
    off_r, sp_r, pp_r = oracle.dispatch_tail_skip(ids, E, tail_from)
    n = int(off_r[E])
    assert np.array_equal(off.cpu().numpy(), off_r)
    assert np.array_equal(sp.cpu().numpy()[:n], sp_r[:n])
    assert np.array_equal(pp.cpu().numpy(), pp_r)
    assert np.all(sp.cpu().numpy()[n:] == -7)   # nothing written past the kept pairs


def _layer_case(w, L, x, tail_from, sample=None):
    from quantized_moe_route_amd.layer import DeviceLayer, alloc_buffers, run_layer
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    T, k, E, d = x.shape[0], w.k, w.n_experts, w.d_model
    b = alloc_buffers(dl, T, k)
    run_layer(dl, torch.from_numpy(x.view(np.int16)).cuda(), b, tail_from=tail_from)
    torch.cuda.synchronize()
    lg = b.logits[:T].cpu().numpy()
    ids_ref, _ = oracle.topk_softmax(lg, k)
    assert np.array_equal(b.ids[:T].cpu().numpy(), ids_ref)
    off_r, sp_r, pp_r = oracle.dispatch_tail_skip(ids_ref, E, tail_from)
    assert np.array_equal(b.offsets.cpu().numpy(), off_r)
    assert np.array_equal(b.pair_pos[:T * k].cpu().numpy(), pp_r)
    rows = np.arange(T) if sample is None else sample
    if sample is None:
        _, _, out_ref = oracle.layer(L, w.fmt, d, w.d_ff, E, k, x, logits=lg, tail_from=tail_from)
    else:
        # the keep set belongs to the whole batch: compose the sampled tokens'
        # output from their kept rows
        keep = oracle.tail_keep(ids_ref, E, tail_from)
        idr = ids_ref[rows]
        re = np.concatenate([idr.ravel(), -np.ones(len(rows), np.int32)]).astype(np.int32)
        rt = np.concatenate([np.repeat(rows, k), rows]).astype(np.int32)
        y = oracle.expert_rows(L, w.fmt, d, w.d_ff, E, x, re, rt, f64=True)
        wr = b.w[:T].cpu().numpy()[rows].astype(np.float64) * keep[idr]
        out_ref = y[len(rows) * k:] + np.einsum("tj,tjd->td", wr, y[:len(rows) * k].reshape(len(rows), k, d))
    err = _rel_err(b.out[:T].cpu().numpy()[rows], out_ref)
    assert err <= TOL, err
    return err, int(off_r[E])


@pytest.mark.parametrize("wid,tail_from", [(1, 6), (2, 6), (0, 1), (5, 6)])
def test_layer_tail_skip_workloads(q, wid, tail_from):
    w = synth.WORKLOADS[wid]
    print(f"workload {w.name} tail_from={tail_from}", flush=True)
    L = synth.gen_layer(w, layer=0)
    x = synth.gen_x(w, layer=0)
    err, kept = _layer_case(w, L, x, tail_from)
    print(f"kept pairs {kept} of {w.T * w.k}, max|err|/rms = {err:.3e}")


@pytest.mark.parametrize("fmt,T,E,k,tail_from", [(2, 300, 64, 8, 4), (1, 40, 512, 10, 6), (1, 12, 64, 8, 2)])
def test_layer_tail_skip_shapes(q, fmt, T, E, k, tail_from):
    """Both expert paths (T <= 16 and above) with dropped groups."""
    w = synth.custom(256, 128, E, k, T, fmt=fmt, zipf_s=1.3 if fmt == 2 else 0.0, wid=960 + T)
    print(f"shape {w} tail_from={tail_from}", flush=True)
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    sample = None if T <= 64 else np.sort(np.random.default_rng(T).choice(T, size=32, replace=False))
    err, kept = _layer_case(w, L, x, tail_from, sample=sample)
    assert kept < T * k
    print(f"kept pairs {kept} of {T * k}, max|err|/rms = {err:.3e}")


@pytest.mark.parametrize("T,tail_from", [(1, 6), (4, 3), (8, 0), (8, 10), (12, 6)])
def test_route_dispatch_tail_skip_equals_two_calls(q, T, tail_from):
    """moe_route_dispatch_tail_skip (one launch up to 8 tokens) writes what
    moe_route then moe_dispatch_tail_skip write, bit for bit."""
    E, k, d = 64, 10, 512
    w = synth.custom(d, 256, E, k, T, fmt=1, zipf_s=1.3, wid=900 + T)
    x = torch.from_numpy(synth.gen_x(w).view(np.int16)).cuda()
    wr = torch.from_numpy(synth.gen_router(w)).cuda()
    n_ws = q.moe_workspace_size(d, 256, E, T, k)
    outs = []
    for fused in (False, True):
        ws = torch.zeros(n_ws + 256, dtype=torch.uint8, device="cuda")
        ws = ws[(-ws.data_ptr()) % 256:][:n_ws]
        lg = torch.full((T, E), 3.0, device="cuda")
        ids = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
        wt = torch.full((T, k), -5.0, device="cuda")
        off = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")
        sp = torch.full((T * k,), -5, dtype=torch.int32, device="cuda")
        pp = torch.full((T * k,), -5, dtype=torch.int32, device="cuda")
        if fused:
            q.moe_route_dispatch_tail_skip(x, wr, None, lg, T, d, E, k, tail_from, ids, wt, off, sp, pp, ws, n_ws)
        else:
            q.moe_route(x, wr, None, lg, T, d, E, k, ids, wt, ws, n_ws)
            q.moe_dispatch_tail_skip(ids, T, E, k, tail_from, off, sp, pp, ws, n_ws)
        torch.cuda.synchronize()
        n = int(off[E].item())
        outs.append([lg.cpu().numpy(), ids.cpu().numpy(), wt.cpu().numpy(), off.cpu().numpy(),
                     sp[:n].cpu().numpy(), pp.cpu().numpy()])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ref_off, ref_sp, ref_pp = oracle.dispatch_tail_skip(outs[1][1], E, tail_from)
    assert np.array_equal(outs[1][3], ref_off) and np.array_equal(outs[1][5], ref_pp)
