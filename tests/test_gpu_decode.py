"""GPU parity, decode / MTP-verify shapes (T <= 16): the HIP path through the
C ABI against the CPU oracle on the same seeded inputs.

Bars: ids, offsets, permutation bit-exact (on identical logits);
float outputs max|gpu - oracle| <= 2e-3 * rms(oracle).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import packing

# the workspace's counter header: 4 KiB for the router's token tiles (and
# the error word), one 128-byte line per 16-column output tile (d <= 16,384)
# for the fused combine, one line per (token tile, 32-expert slice) for the
# router
WS_HEADER = 4096 + 1024 * 128 + 16 * 32 * 128
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def q():
    _need_gpu()
    import quantized_moe_route_amd as q
    return q


def _rel_err(gpu, ref):
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / rms)


def _upload(L, w):
    from quantized_moe_route_amd.layer import DeviceLayer
    return DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)


def _x_dev(x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda()


def _run(q, dl, w, x_bits, T=None, logits=None):
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    T = x_bits.shape[0] if T is None else T
    b = alloc_buffers(dl, T, w.k)
    if logits is not None:
        b.logits[:T].copy_(torch.from_numpy(logits))
    run_layer(dl, _x_dev(x_bits), b, logits_in=logits is not None)
    torch.cuda.synchronize()
    return b


def _check_layer(q, w, L, x_bits, b):
    """Full parity of one layer run against the oracle, routing on GPU logits."""
    T, k, E, d = x_bits.shape[0], w.k, w.n_experts, w.d_model
    lg_gpu = b.logits[:T].cpu().numpy()
    lg_ref = oracle.router_logits(x_bits, L.router, L.bias)
    assert _rel_err(lg_gpu, lg_ref) <= 1e-5
    ids_ref, w_ref = oracle.topk_softmax(lg_gpu, k)
    ids = b.ids[:T].cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    assert np.max(np.abs(b.w[:T].cpu().numpy() - w_ref)) <= 1e-6
    off_ref, sp_ref, pp_ref = oracle.dispatch(ids_ref, E)
    assert np.array_equal(b.offsets.cpu().numpy(), off_ref)
    assert np.array_equal(b.sorted_pair[:T * k].cpu().numpy(), sp_ref)
    assert np.array_equal(b.pair_pos[:T * k].cpu().numpy(), pp_ref)
    flat = ids_ref.ravel()
    re = np.concatenate([flat[sp_ref], -np.ones(T, np.int32)]).astype(np.int32)
    rt = np.concatenate([sp_ref // k, np.arange(T)]).astype(np.int32)
    y_ref = oracle.expert_rows(L, w.fmt, d, w.d_ff, E, x_bits, re, rt)
    P = T * k
    assert _rel_err(b.y_pairs[:P].cpu().numpy(), y_ref[:P]) <= TOL
    assert _rel_err(b.y_shared[:T].cpu().numpy(), y_ref[P:]) <= TOL
    _, _, out_ref = oracle.layer(L, w.fmt, d, w.d_ff, E, k, x_bits, logits=lg_gpu)
    err = _rel_err(b.out[:T].cpu().numpy(), out_ref)
    assert err <= TOL, err
    return err


@pytest.mark.parametrize("wid,layer", [(0, 0), (1, 0), (2, 0), (2, 23), (2, 47), (5, 0)])
def test_workload_layer_parity(q, wid, layer):
    """Every token of the layer against the oracle; for the 48-layer MTP
    stack, the first, a middle and the last layer (each has its own weights
    and Zipf router bias)."""
    w = synth.WORKLOADS[wid]
    print(f"workload {w.name} layer {layer}", flush=True)
    L = synth.gen_layer(w, layer=layer)
    x = synth.gen_x(w, layer=layer)
    dl = _upload(L, w)
    b = _run(q, dl, w, x)
    err = _check_layer(q, w, L, x, b)
    print(f"max|err|/rms = {err:.3e}")


@pytest.mark.parametrize("fmt,T,E,k,d,f", [
    (1, 1, 16, 2, 256, 128), (2, 2, 64, 8, 256, 256), (1, 3, 64, 8, 384, 128),
    (2, 5, 32, 4, 128, 384), (1, 16, 16, 2, 256, 128), (2, 12, 64, 10, 256, 128),
    (1, 9, 1, 1, 128, 128), (2, 4, 8, 8, 128, 128), (1, 16, 512, 10, 128, 128),
    # 321 expert groups; d_ff = 1536: several down batches
    (2, 16, 1024, 20, 128, 128), (1, 2, 16, 2, 128, 1536),
])
def test_shape_sweep_parity(q, fmt, T, E, k, d, f):
    w = synth.custom(d, f, E, k, T, fmt=fmt, zipf_s=1.3 if fmt == 2 else 0.0, wid=200 + T)
    print(f"shape {w}", flush=True)
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    b = _run(q, _upload(L, w), w, x)
    _check_layer(q, w, L, x, b)


@pytest.mark.parametrize("T,E,k", [(8, 512, 10), (5, 64, 64), (3, 1024, 32), (4, 16, 16),
                                   (6, 100, 33), (257, 512, 10), (2, 1024, 1024)])
def test_route_logits_input_ties(q, T, E, k):
    """Forced ties (integer logits, signed zeros, all-equal rows): ids bit-exact,
    for the ranking selection (k <= 32) and the serial one (k > 32)."""
    rng = np.random.default_rng(3 + T + E + k)
    lg = np.round(rng.standard_normal((T, E)) * 2).astype(np.float32)
    lg[1] = 0.0
    lg[1, ::2] = -0.0
    if T > 2:
        lg[2] = 7.0
    if T > 3:
        lg[3, E // 4:E // 4 + min(10, E // 2)] = 50.0
    lg_d = torch.from_numpy(lg).cuda()
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    n_ws = q.moe_workspace_size(2048, 128, E, T, k)
    ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    q.moe_route(None, None, None, lg_d, T, 2048, E, k, ids, wt, ws, n_ws)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.topk_softmax(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6


@pytest.mark.parametrize("T,E,k,d", [(8, 1024, 32, 256), (7, 300, 40, 384), (1, 33, 33, 128),
                                     (8, 512, 10, 2048), (9, 512, 10, 2048), (20, 1000, 70, 256),
                                     (63, 300, 40, 384), (100, 1024, 32, 128), (128, 512, 10, 2048)])
def test_route_small_path_shapes(q, T, E, k, d):
    """One-launch router (T <= 128, tiles of 8 tokens, the last one ragged):
    logits within tolerance, ids bit-exact on them."""
    rng = np.random.default_rng(T * E + k)
    x = synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    wr = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    ws_bytes = q.moe_workspace_size(d, 128, E, T, k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    lg = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, device="cuda")
    c = lambda a: torch.from_numpy(a).cuda()
    for rep in range(2):      # second call checks the self-resetting arrival counter
        q.moe_route(c(x.view(np.int16)), c(wr), c(bias), lg, T, d, E, k, ids, wt, ws, ws_bytes)
        torch.cuda.synchronize()
        lg_h = lg.cpu().numpy()
        assert _rel_err(lg_h, oracle.router_logits(x, wr, bias)) <= 1e-5
        ids_ref, w_ref = oracle.topk_softmax(lg_h, k)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6


@pytest.mark.parametrize("T,E,k,d", [(1, 512, 10, 2048), (4, 512, 10, 512), (8, 1024, 64, 256),
                                     (1, 64, 40, 128), (1, 1024, 64, 128)])
def test_route_small_exact_ties(q, T, E, k, d):
    """One-launch router and listing on logits with exact ties: the router
    columns are 8 distinct ones repeated, so runs of experts share a logit bit
    for bit and the pruning bound ties across groups.  ids (lower expert first
    on a tie), weights and the listing against the oracle on the GPU's logits."""
    rng = np.random.default_rng(7 * T + E + k)
    x = synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    cols = rng.integers(0, 8, E)
    wr = np.ascontiguousarray((rng.standard_normal((d, 8)) / np.sqrt(d)).astype(np.float32)[:, cols])
    ws_bytes = q.moe_workspace_size(d, 128, E, T, k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    lg = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    c = lambda a: torch.from_numpy(a).cuda()
    q.moe_route_dispatch(c(x.view(np.int16)), c(wr), None, lg, T, d, E, k, ids, wt, off, sp, pp, ws, ws_bytes)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    for j in range(8):   # equal columns give equal logits
        same = lg_h[:, cols == j]
        assert same.size == 0 or np.array_equal(same, np.repeat(same[:, :1], same.shape[1], axis=1))
    ids_ref, w_ref = oracle.topk_softmax(lg_h, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6
    off_ref, sp_ref, pp_ref = oracle.dispatch(ids_ref, E)
    assert np.array_equal(off.cpu().numpy(), off_ref) and np.array_equal(sp.cpu().numpy(), sp_ref)
    assert np.array_equal(pp.cpu().numpy(), pp_ref)


@pytest.mark.parametrize("T,E,k,d", [(300, 300, 40, 384), (257, 1000, 70, 256), (1000, 64, 8, 128),
                                     (513, 17, 3, 2048), (129, 512, 10, 2048)])
def test_route_gemm_path_shapes(q, T, E, k, d):
    """Router matrix-core path (T > 128) at ragged shapes: token and expert
    tiles with tails, E not a multiple of 64, and k > 64 (top-k through LDS)."""
    rng = np.random.default_rng(T * E + k + d)
    x = synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    wr = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    ws_bytes = q.moe_workspace_size(d, 128, E, T, k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    lg = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, device="cuda")
    c = lambda a: torch.from_numpy(a).cuda()
    q.moe_route(c(x.view(np.int16)), c(wr), c(bias), lg, T, d, E, k, ids, wt, ws, ws_bytes)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    assert _rel_err(lg_h, oracle.router_logits(x, wr, bias)) <= 1e-5
    ids_ref, w_ref = oracle.topk_softmax(lg_h, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(wt.cpu().numpy() - w_ref)) <= 1e-6


@pytest.mark.parametrize("T,E,k,skew", [
    (1, 512, 10, 0), (4, 512, 10, 1), (100, 64, 8, 0), (512, 512, 8, 0), (8192, 512, 10, 0),
    (8192, 512, 10, 2), (300, 1024, 16, 0), (65, 16, 16, 0), (1000, 1, 1, 0),
])
def test_dispatch_parity(q, T, E, k, skew):
    rng = np.random.default_rng(T * 7 + E + k)
    if skew == 0:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    elif skew == 1:
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    else:  # Zipf-like skew: many tokens share a few experts
        pr = 1.0 / np.arange(1, E + 1) ** 1.3
        pr /= pr.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=pr) for _ in range(T)]).astype(np.int32)
    ws_bytes = q.moe_workspace_size(128, 128, E, T, k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    q.moe_dispatch(torch.from_numpy(ids).cuda(), T, E, k, off, sp, pp, ws, ws_bytes)
    torch.cuda.synchronize()
    o_ref, sp_ref, pp_ref = oracle.dispatch(ids, E)
    assert np.array_equal(off.cpu().numpy(), o_ref)
    assert np.array_equal(sp.cpu().numpy(), sp_ref)
    assert np.array_equal(pp.cpu().numpy(), pp_ref)


def test_combine_parity(q):
    rng = np.random.default_rng(9)
    T, k, d = 33, 10, 2048
    P = T * k
    yp = rng.standard_normal((P, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32)
    pp = rng.permutation(P).astype(np.int32)
    wt = rng.random((T, k)).astype(np.float32)
    out = torch.empty(T, d, device="cuda")
    c = lambda a: torch.from_numpy(a).cuda()
    q.moe_combine(c(yp), c(ys), c(pp), c(wt), T, k, d, out)
    torch.cuda.synchronize()
    ref = oracle.combine(yp, ys, pp, wt, T, k, d)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-5 * np.sqrt(np.mean(ref.astype(np.float64) ** 2))


def test_identical_experts_and_zero_experts(q):
    """Pins that carry over to the GPU: identical routed experts make the output
    independent of routing; zero routed weights leave the shared expert."""
    from quantized_moe_route_amd.layer import DeviceLayer, alloc_buffers, run_layer
    rng = np.random.default_rng(12)
    d, f, E, k, T = 256, 128, 16, 4, 6
    for mode in ("same", "zero"):
        mats = {}
        for name, (n, rows, K) in {"gate": (E, f, d), "up": (E, f, d), "down": (E, d, f),
                                   "sh_gate": (1, f, d), "sh_up": (1, f, d), "sh_down": (1, d, f)}.items():
            m, _ = packing.random_mat(rng, 1, n, rows, K, zero=(mode == "zero" and n == E))
            if mode == "same" and n == E:
                for pl in ("lo", "scale", "min"):
                    a = getattr(m, pl)
                    per = a.size // E
                    a[:] = np.tile(a[:per], E)
            mats[name] = m

        class H:
            pass
        for n_, m in mats.items():
            setattr(H, n_, m)
        x = synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
        outs = []
        for s in range(2):
            lg = rng.standard_normal((T, E)).astype(np.float32)
            dl = DeviceLayer.from_host(1, d, f, E, H, np.zeros((d, E), np.float32))
            b = alloc_buffers(dl, T, k)
            b.logits.copy_(torch.from_numpy(lg))
            run_layer(dl, _x_dev(x), b, logits_in=True)
            torch.cuda.synchronize()
            outs.append(b.out.cpu().numpy())
            _, _, ref = oracle.layer(H, 1, d, f, E, k, x, logits=lg)
            assert _rel_err(outs[-1], ref) <= TOL
        if mode == "same":
            assert _rel_err(outs[0], outs[1]) <= TOL


def test_repeatable_bitwise(q):
    w = synth.WORKLOADS[0]
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    dl = _upload(L, w)
    b1 = _run(q, dl, w, x)
    o1, i1 = b1.out.cpu().numpy().copy(), b1.ids.cpu().numpy().copy()
    b2 = _run(q, dl, w, x)
    assert np.array_equal(o1, b2.out.cpu().numpy()) and np.array_equal(i1, b2.ids.cpu().numpy())


def test_token_independence_gpu(q):
    """A T=4 batch equals four T=1 runs within tolerance (MTP verify sanity)."""
    w = synth.custom(256, 128, 16, 2, 4, wid=300)
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    dl = _upload(L, w)
    b = _run(q, dl, w, x)
    full = b.out.cpu().numpy().copy()
    for t in range(4):
        bt = _run(q, dl, w, x[t:t + 1])
        assert _rel_err(bt.out[:1].cpu().numpy(), full[t:t + 1]) <= TOL


def test_t_zero_is_noop(q):
    n_ws = q.moe_workspace_size(256, 128, 16, 1, 2)
    ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    lg = torch.full((1, 16), 3.0, device="cuda")
    ids = torch.full((1, 2), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((1, 2), -7.0, device="cuda")
    x = torch.zeros(1, 256, dtype=torch.int16, device="cuda")
    wr = torch.zeros(256, 16, device="cuda")
    q.moe_route(x, wr, None, lg, 0, 256, 16, 2, ids, wt, ws, n_ws)
    torch.cuda.synchronize()
    assert torch.all(ids == -7) and torch.all(wt == -7.0) and torch.all(lg == 3.0)


@pytest.mark.parametrize("T,fmt", [(4, 2), (1, 1), (16, 2)])
def test_back_to_back_calls_share_workspace(q, T, fmt):
    """Consecutive layers on one workspace: the in-kernel ticket and per-group
    counters must be back at zero after every call (the workspace's
    counter header reads all zero), and every layer matches the oracle."""
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    w = synth.custom(256, 128, 64, 8, T, fmt=fmt, zipf_s=1.3, wid=310 + T)
    print(f"shape {w}", flush=True)
    L = synth.gen_layer(w)
    dl = _upload(L, w)
    b = alloc_buffers(dl, w.T, w.k)
    for step in range(3):
        x = synth.gen_x(w, stream=step)
        run_layer(dl, _x_dev(x), b)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(b.ws[:WS_HEADER])) == 0, step
        _check_layer(q, w, L, x, b)


def test_graph_replay_matches_eager(q):
    """The layer captured once in a HIP graph and replayed, with eager calls
    and host synchronisations between replays: every replay equals the eager
    result bitwise."""
    from quantized_moe_route_amd import hip
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    w = synth.custom(256, 256, 64, 8, 4, fmt=1, wid=320)
    L = synth.gen_layer(w)
    dl = _upload(L, w)
    stream = torch.cuda.Stream()
    xs = [_x_dev(synth.gen_x(w, stream=s)) for s in range(3)]
    x_in = xs[0].clone()
    with torch.cuda.stream(stream):
        b = alloc_buffers(dl, w.T, w.k, stream=stream)
    torch.cuda.synchronize()
    with hip.Graph(stream.cuda_stream) as g:
        run_layer(dl, x_in, b, stream=stream.cuda_stream)
    for rep in range(3):
        x_in.copy_(xs[rep])
        torch.cuda.synchronize()
        # eager reference on separate buffers
        be = alloc_buffers(dl, w.T, w.k)
        run_layer(dl, xs[rep], be)
        torch.cuda.synchronize()
        g.launch()
        hip.stream_synchronize(stream.cuda_stream)
        assert torch.equal(b.out, be.out) and torch.equal(b.ids, be.ids), rep


@pytest.mark.parametrize("T,E,k,d", [(1, 512, 10, 2048), (4, 512, 10, 2048), (8, 1024, 64, 256),
                                     (3, 16, 2, 128), (9, 512, 10, 256), (5, 300, 70, 128)])
def test_route_dispatch_equals_separate_calls(q, T, E, k, d):
    """moe_route_dispatch writes what moe_route then moe_dispatch write, bit
    for bit: one launch for one tile (T <= 8, k <= 64), the two calls
    otherwise (T = 9; k = 70)."""
    rng = np.random.default_rng(T * 11 + E + k)
    x = torch.from_numpy(synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
                         .view(np.int16)).cuda()
    wr = torch.from_numpy((rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)).cuda()
    bias = torch.from_numpy(rng.standard_normal(E).astype(np.float32)).cuda()
    ws_bytes = q.moe_workspace_size(d, 128, E, T, k)
    outs = []
    for fused in (False, True):
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        lg = torch.full((T, E), -5.0, device="cuda")
        ids = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
        wt = torch.full((T, k), -5.0, device="cuda")
        off = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")
        sp = torch.full((T * k,), -5, dtype=torch.int32, device="cuda")
        pp = torch.full((T * k,), -5, dtype=torch.int32, device="cuda")
        for rep in range(2):   # the second call checks the arrival counter is back at zero
            if fused:
                q.moe_route_dispatch(x, wr, bias, lg, T, d, E, k, ids, wt, off, sp, pp, ws, ws_bytes)
            else:
                q.moe_route(x, wr, bias, lg, T, d, E, k, ids, wt, ws, ws_bytes)
                q.moe_dispatch(ids, T, E, k, off, sp, pp, ws, ws_bytes)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:WS_HEADER])) == 0
        outs.append([t.cpu().numpy() for t in (lg, ids, wt, off, sp, pp)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    off_ref, sp_ref, pp_ref = oracle.dispatch(outs[1][1], E)
    assert np.array_equal(outs[1][3], off_ref) and np.array_equal(outs[1][4], sp_ref)
    assert np.array_equal(outs[1][5], pp_ref)


@pytest.mark.parametrize("wid", [1, 2])
def test_workload_layer_parity_fused_route_dispatch(q, wid):
    w = synth.WORKLOADS[wid]
    L = synth.gen_layer(w, layer=0)
    x = synth.gen_x(w, layer=0)
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    dl = _upload(L, w)
    b = alloc_buffers(dl, w.T, w.k)
    run_layer(dl, _x_dev(x), b, fused=True)
    torch.cuda.synchronize()
    _check_layer(q, w, L, x, b)
