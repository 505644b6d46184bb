"""GPU: moe_expert_ffn_noalloc (no workspace argument; the library's fixed
device scratch) against moe_expert_ffn with a caller workspace, through the
C ABI.  The two run the same kernels, so y_pairs and y_shared must agree bit
for bit.  Two calls in a row, the second with fewer tokens (the scratch
keeps the first call's contents), then sizes beyond the scratch's maximum,
which must be rejected before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_route_amd as q
    return q


def _routed(q, dl, w, x, T):
    from quantized_moe_route_amd.layer import alloc_buffers
    b = alloc_buffers(dl, T, w.k)
    q.moe_route(x, dl.router, dl.bias, b.logits, T, w.d_model, w.n_experts, w.k, b.ids, b.w, b.ws, b.ws_bytes)
    q.moe_dispatch(b.ids, T, w.n_experts, w.k, b.offsets, b.sorted_pair, b.pair_pos, b.ws, b.ws_bytes)
    return b


@pytest.mark.parametrize("fmt", [1, 2])
def test_noalloc_matches_workspace_call_twice(q, fmt):
    from quantized_moe_route_amd.layer import DeviceLayer
    w = synth.custom(2048, 768, 512, 10, 16, fmt=fmt, zipf_s=1.1 if fmt == 2 else 0.0, wid=900 + fmt)
    L = synth.gen_layer(w)
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    for T in (16, 4, 1):   # each call smaller than the one before
        print(f"fmt {fmt} T {T}", flush=True)
        x = torch.from_numpy(synth.gen_x(w, T=T, seed=T).view(np.int16)).cuda()
        b = _routed(q, dl, w, x, T)
        q.moe_expert_ffn(dl.struct, x, T, w.k, b.offsets, b.sorted_pair, b.y_pairs, b.y_shared, b.ws, b.ws_bytes)
        torch.cuda.synchronize()
        ref_p, ref_s = b.y_pairs[:T * w.k].clone(), b.y_shared[:T].clone()
        b.y_pairs.fill_(float("nan"))
        b.y_shared.fill_(float("nan"))
        q.moe_expert_ffn_noalloc(dl.struct, x, T, w.k, b.offsets, b.sorted_pair, b.y_pairs, b.y_shared)
        torch.cuda.synchronize()
        assert torch.equal(b.y_pairs[:T * w.k], ref_p)
        assert torch.equal(b.y_shared[:T], ref_s)


def test_noalloc_on_a_side_stream(q):
    """Ordered on a non-default stream: same result."""
    from quantized_moe_route_amd.layer import DeviceLayer
    w = synth.custom(256, 128, 16, 2, 4, fmt=1, wid=910)
    L = synth.gen_layer(w)
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    x = torch.from_numpy(synth.gen_x(w).view(np.int16)).cuda()
    b = _routed(q, dl, w, x, w.T)
    q.moe_expert_ffn(dl.struct, x, w.T, w.k, b.offsets, b.sorted_pair, b.y_pairs, b.y_shared, b.ws, b.ws_bytes)
    torch.cuda.synchronize()
    ref_p, ref_s = b.y_pairs.clone(), b.y_shared.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b.y_pairs.fill_(0.0)
        b.y_shared.fill_(0.0)
        q.moe_expert_ffn_noalloc(dl.struct, x, w.T, w.k, b.offsets, b.sorted_pair, b.y_pairs, b.y_shared, s)
    torch.cuda.synchronize()
    assert torch.equal(b.y_pairs, ref_p) and torch.equal(b.y_shared, ref_s)


def test_noalloc_rejects_sizes_beyond_the_scratch(q):
    from quantized_moe_route_amd.layer import DeviceLayer
    w = synth.custom(256, 128, 16, 2, 4, fmt=1, wid=920)
    L = synth.gen_layer(w)
    dl = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias)
    A = 4096
    # more than 16 tokens: the grouped GEMM path needs a caller workspace
    assert q.moe_expert_ffn_noalloc(dl.struct, A, 17, 2, A, A, A, A, check=False) == q.MOE_ERR_UNSUPPORTED
    # a shape whose scratch exceeds 8 MiB: 16 tokens x top-64 at d_ff = 16384
    import ctypes as C
    big = q.moe_layer.from_buffer_copy(dl.struct)
    big.d_ff = 16384
    big.n_experts = 64
    assert q.moe_expert_ffn_noalloc(big, A, 16, 64, A, A, A, A, check=False) == q.MOE_ERR_UNSUPPORTED
    assert q.moe_expert_ffn_noalloc(dl.struct, A, 0, 2, A, A, A, A, check=False) == q.MOE_OK   # T = 0
