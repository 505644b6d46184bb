"""GPU: moe_expert_ffn_combine against moe_expert_ffn then moe_combine.

With T <= 4 the down kernel merges each 16-column output tile itself (the
last workgroup of the tile to finish), so the fused call must write the same
y_pairs, y_shared and out as the two calls, bit for bit, leave the
workspace's counter header at zero, and work back to back on one workspace
and replayed from a HIP graph.  Above 4 tokens it enqueues the two calls.
The layer output is also checked against the oracle (2e-3 * rms(out)).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
# the workspace's counter header: 4 KiB for the router's token tiles (and
# the error word), one 128-byte line per 16-column output tile (d <= 16,384)
# for the fused combine, one line per (token tile, 32-expert slice) for the
# router
WS_HEADER = 4096 + 1024 * 128 + 16 * 32 * 128


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_route_amd as q
    return q


def _setup(w):
    from quantized_moe_route_amd.layer import DeviceLayer, alloc_buffers
    L = synth.gen_layer(w)
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    return L, dl, alloc_buffers(dl, w.T, w.k)


def _xdev(x):
    return torch.from_numpy(x.view(np.int16)).cuda()


def _two_calls_then_fused(q, w, dl, b, xd, tail_from=None):
    """Reference (route, dispatch, expert FFN, combine), then the fused call
    on the same routing into poisoned outputs; returns (ref, fused) tuples of
    (y_pairs kept rows, y_shared, out)."""
    from quantized_moe_route_amd.layer import run_layer
    T, E = w.T, w.n_experts
    run_layer(dl, xd, b, tail_from=tail_from)
    torch.cuda.synchronize()
    n = int(b.offsets[E].item())
    ref = (b.y_pairs[:n].clone(), b.y_shared[:T].clone(), b.out[:T].clone())
    for t in (b.y_pairs, b.y_shared, b.out):
        t.fill_(float("nan"))
    q.moe_expert_ffn_combine(dl.struct, xd, T, w.k, b.offsets, b.sorted_pair, b.pair_pos, b.w,
                             b.y_pairs, b.y_shared, b.out, b.ws, b.ws_bytes)
    torch.cuda.synchronize()
    return ref, (b.y_pairs[:n], b.y_shared[:T], b.out[:T])


SHAPES = [
    # (fmt, T, E, k, d, f): the full decode layer, small batches of each
    # down-tile form up to 4 tokens, and sizes above 4 tokens (two calls)
    (1, 1, 512, 10, 2048, 768),
    (2, 4, 512, 10, 2048, 768),
    (1, 2, 64, 8, 256, 128),
    (2, 8, 16, 4, 512, 256),
    (1, 16, 64, 8, 256, 128),
    (2, 16, 1024, 20, 128, 128),
    (1, 17, 16, 2, 256, 128),
    (2, 100, 64, 8, 256, 256),
]


@pytest.mark.parametrize("fmt,T,E,k,d,f", SHAPES)
def test_fused_equals_two_calls(q, fmt, T, E, k, d, f):
    w = synth.custom(d, f, E, k, T, fmt=fmt, zipf_s=1.3 if fmt == 2 else 0.0, wid=800 + T)
    print(f"shape {w}", flush=True)
    L, dl, b = _setup(w)
    x = synth.gen_x(w)
    ref, got = _two_calls_then_fused(q, w, dl, b, _xdev(x))
    for name, r, g in zip(("y_pairs", "y_shared", "out"), ref, got):
        assert torch.equal(r, g), name
    assert int(torch.count_nonzero(b.ws[:WS_HEADER])) == 0
    lg = b.logits[:T].cpu().numpy()
    _, _, out_ref = oracle.layer(L, w.fmt, d, f, E, k, x, logits=lg)
    out_ref = np.asarray(out_ref, np.float64)
    err = float(np.max(np.abs(got[2].cpu().numpy() - out_ref)) / np.sqrt(np.mean(out_ref ** 2)))
    print(f"max|err|/rms = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("T", [1, 4])
def test_fused_with_tail_skip(q, T):
    """Dropped pairs (pair_pos -1) add nothing, as in moe_combine."""
    w = synth.custom(512, 256, 64, 8, T, fmt=1, wid=830 + T)
    L, dl, b = _setup(w)
    ref, got = _two_calls_then_fused(q, w, dl, b, _xdev(synth.gen_x(w)), tail_from=3)
    if T == 1:   # one token: every pick from rank 3 on is dropped
        assert int((b.pair_pos[:w.k] < 0).sum().item()) == w.k - 3
    for name, r, g in zip(("y_pairs", "y_shared", "out"), ref, got):
        assert torch.equal(r, g), name


def test_fused_back_to_back_one_workspace(q):
    """T = 4, 1, 16, 8 in a row on one workspace: the tile counters must be
    back at zero after every call."""
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    w16 = synth.custom(256, 128, 64, 8, 16, fmt=2, zipf_s=1.3, wid=850)
    L, dl, b = _setup(w16)
    for T in (4, 1, 16, 8):
        w = synth.custom(256, 128, 64, 8, T, fmt=2, zipf_s=1.3, wid=850)
        bt = alloc_buffers(dl, T, w.k)
        xd = _xdev(synth.gen_x(w, seed=T))
        run_layer(dl, xd, bt)
        torch.cuda.synchronize()
        ref = bt.out[:T].clone()
        bt.out.fill_(float("nan"))
        # the fused call on the shared workspace b.ws (sized for T = 16)
        q.moe_expert_ffn_combine(dl.struct, xd, T, w.k, bt.offsets, bt.sorted_pair, bt.pair_pos, bt.w,
                                 bt.y_pairs, bt.y_shared, bt.out, b.ws, b.ws_bytes)
        torch.cuda.synchronize()
        assert torch.equal(bt.out[:T], ref), T
        assert int(torch.count_nonzero(b.ws[:WS_HEADER])) == 0, T


@pytest.mark.parametrize("T", [1, 4])
def test_fused_graph_replay(q, T):
    """route_dispatch + expert_ffn_combine captured once; three replays with
    new inputs and eager work between them, each equal to the eager layer."""
    from quantized_moe_route_amd import hip
    from quantized_moe_route_amd.layer import run_layer
    w = synth.custom(512, 256, 64, 8, T, fmt=1, wid=870)
    L, dl, b = _setup(w)
    main = torch.cuda.Stream()
    sh = main.cuda_stream
    xin = torch.empty_like(_xdev(synth.gen_x(w)))
    torch.cuda.synchronize()
    with hip.Graph(sh) as g:
        run_layer(dl, xin, b, stream=sh, fused=True, fuse_combine=True)
    for rep in range(3):
        xr = _xdev(synth.gen_x(w, seed=rep + 5))
        run_layer(dl, xr, b, stream=sh)
        hip.stream_synchronize(sh)
        ref = b.out[:w.T].clone()
        xin.copy_(xr)
        b.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        hip.stream_synchronize(sh)
        assert torch.equal(b.out[:w.T], ref), rep
