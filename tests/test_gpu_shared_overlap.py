"""GPU: the shared expert computed beside routing.

moe_shared_ffn (the shared expert; it needs only x) runs on a second stream
while routing runs; moe_routed_ffn runs after routing; the streams join
before moe_combine.  Bars:
  - moe_routed_ffn's y_pairs and moe_shared_ffn's y_shared equal those of
    moe_expert_ffn bit for bit (same kernels, same per-row arithmetic), on
    the single-token, small-batch, mid-size and large-batch paths, and each
    call leaves the other half's output untouched;
  - the overlapped layer's out equals the one-stream layer's bit for bit,
    eagerly and replayed from a HIP graph with the fork and join captured,
    and matches the oracle within 2e-3 * rms(out).
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


def _setup(w):
    from quantized_moe_route_amd.layer import DeviceLayer, alloc_buffers
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    b = alloc_buffers(dl, w.T, w.k)
    return L, x, dl, b, torch.from_numpy(x.view(np.int16)).cuda()


SPLIT_SHAPES = [
    # (fmt, T, E, k, d, f): T = 1 at the full layer size, the small-batch
    # path (T <= 16), the mid-size build (17 .. 2,048) and the large build
    (1, 1, 512, 10, 2048, 768),
    (2, 4, 512, 10, 2048, 768),
    (1, 16, 64, 8, 256, 128),
    (2, 17, 16, 2, 256, 128),
    (1, 300, 64, 8, 256, 256),
    (2, 2049, 32, 4, 128, 128),
    (1, 2500, 16, 2, 256, 128),
]


@pytest.mark.parametrize("fmt,T,E,k,d,f", SPLIT_SHAPES)
def test_split_ffn_equals_expert_ffn(q, fmt, T, E, k, d, f):
    from quantized_moe_route_amd.layer import run_layer
    w = synth.custom(d, f, E, k, T, fmt=fmt, zipf_s=1.3 if fmt == 2 else 0.0, wid=700 + T)
    print(f"shape {w}", flush=True)
    L, x, dl, b, xd = _setup(w)
    run_layer(dl, xd, b)
    torch.cuda.synchronize()
    n = int(b.offsets[E].item())
    yp_ref, ysh_ref = b.y_pairs[:n].clone(), b.y_shared[:T].clone()
    nan = float("nan")
    b.y_pairs.fill_(nan)
    b.y_shared.fill_(nan)
    q.moe_routed_ffn(dl.struct, xd, T, k, b.offsets, b.sorted_pair, b.y_pairs, b.ws, b.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(b.y_pairs[:n], yp_ref)
    assert torch.isnan(b.y_shared).all(), "moe_routed_ffn wrote y_shared"
    b.y_pairs.fill_(nan)
    q.moe_shared_ffn(dl.struct, xd, T, b.y_shared, b.ws_sh, b.ws_sh_bytes)
    torch.cuda.synchronize()
    assert torch.equal(b.y_shared[:T], ysh_ref)
    assert torch.isnan(b.y_pairs).all(), "moe_shared_ffn wrote y_pairs"


@pytest.mark.parametrize("wid", [1, 2])
def test_overlapped_layer_eager(q, wid):
    """Decode (T=1, Q2) and MTP verify (T=4, Q3 Zipf 1.1) layers at full size."""
    from quantized_moe_route_amd.layer import SideStream, run_layer
    w = synth.WORKLOADS[wid]
    print(f"workload {w.name}", flush=True)
    L, x, dl, b, xd = _setup(w)
    main = torch.cuda.Stream()
    sh = main.cuda_stream
    run_layer(dl, xd, b, stream=sh, fused=True)
    torch.cuda.synchronize()
    ref = b.out[:w.T].clone()
    b.out.fill_(float("nan"))
    b.y_shared.fill_(float("nan"))
    run_layer(dl, xd, b, stream=sh, fused=True, side=SideStream())
    torch.cuda.synchronize()
    assert torch.equal(b.out[:w.T], ref)
    lg = b.logits[:w.T].cpu().numpy()
    _, _, out_ref = oracle.layer(L, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x, logits=lg)
    out_ref = np.asarray(out_ref, np.float64)
    err = float(np.max(np.abs(b.out[:w.T].cpu().numpy() - out_ref)) / np.sqrt(np.mean(out_ref ** 2)))
    print(f"max|err|/rms = {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt,T,E,k,d,f", [(1, 1, 64, 8, 512, 256), (2, 40, 32, 4, 256, 128)])
def test_overlapped_layer_graph_replay(q, fmt, T, E, k, d, f):
    """The fork and join captured in a HIP graph; every replay, with eager
    work and a new input between replays, equals the one-stream layer."""
    from quantized_moe_route_amd import hip
    from quantized_moe_route_amd.layer import SideStream, run_layer
    w = synth.custom(d, f, E, k, T, fmt=fmt, wid=760 + T)
    print(f"shape {w}", flush=True)
    L, x, dl, b, xd = _setup(w)
    main = torch.cuda.Stream()
    sh = main.cuda_stream
    side = SideStream()
    xin = torch.empty_like(xd)
    torch.cuda.synchronize()
    with hip.Graph(sh) as g:
        run_layer(dl, xin, b, stream=sh, fused=True, side=side)
    for rep in range(3):
        xr = torch.from_numpy(synth.gen_x(w, seed=rep + 1).view(np.int16)).cuda()
        run_layer(dl, xr, b, stream=sh)
        hip.stream_synchronize(sh)
        ref = b.out[:T].clone()
        xin.copy_(xr)
        b.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        hip.stream_synchronize(sh)
        assert torch.equal(b.out[:T], ref), f"replay {rep}"
