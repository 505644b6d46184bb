"""Device-side holder for one MoE layer and the buffers of one call sequence.

Marshalling only: it owns torch device tensors (weights, router, outputs,
workspaces) and calls the entry points in order, on one stream or with the
shared expert on a second one.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (MOE_FMT_Q2_B32, hip, make_layer, moe_combine, moe_dispatch, moe_dispatch_tail_skip,
               moe_expert_ffn, moe_expert_ffn_combine, moe_route, moe_route_dispatch,
               moe_route_dispatch_tail_skip, moe_routed_ffn, moe_shared_ffn, moe_workspace_init,
               moe_workspace_size)

MATS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")


def _dev(a, device, dtype=None):
    if a is None:
        return None
    t = torch.as_tensor(a)
    if dtype is not None:
        t = t.view(dtype) if t.dtype.itemsize == torch.empty((), dtype=dtype).itemsize else t.to(dtype)
    return t.to(device).contiguous()


class DeviceLayer:
    """Packed planes of the six expert matrices plus router weights, on device.

    `planes[name]` = (lo uint8, hi uint8|None, scale int16 (fp16 bits), min int16|None).
    """

    def __init__(self, fmt, d_model, d_ff, n_experts, planes: dict, router, bias=None):
        self.fmt, self.d_model, self.d_ff, self.n_experts = fmt, d_model, d_ff, n_experts
        self.planes = planes
        self.router = router
        self.bias = bias
        self.struct = make_layer(fmt, d_model, d_ff, n_experts, planes)

    @classmethod
    def from_host(cls, fmt, d_model, d_ff, n_experts, host, router, bias=None, device="cuda"):
        """host: object with attributes gate..sh_down, each having lo/hi/scale/min
        numpy arrays (hi/min may be None)."""
        import numpy as np

        planes = {}
        for n in MATS:
            m = getattr(host, n)
            conv = lambda a, dt: None if a is None else torch.from_numpy(
                np.ascontiguousarray(a).view(dt)).to(device)
            planes[n] = (conv(m.lo, np.uint8), conv(m.hi, np.uint8), conv(m.scale, np.int16),
                         conv(m.min, np.int16))
        r = torch.from_numpy(np.ascontiguousarray(router, dtype=np.float32)).to(device)
        b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(device)
        return cls(fmt, d_model, d_ff, n_experts, planes, r, b)


@dataclasses.dataclass
class Buffers:
    T: int
    k: int
    logits: torch.Tensor
    ids: torch.Tensor
    w: torch.Tensor
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    y_pairs: torch.Tensor
    y_shared: torch.Tensor
    out: torch.Tensor
    ws: torch.Tensor
    ws_bytes: int
    ws_sh: torch.Tensor          # the shared expert's own workspace, for moe_shared_ffn beside routing
    ws_sh_bytes: int


def alloc_buffers(layer: DeviceLayer, T: int, k: int, device="cuda", stream=None) -> Buffers:
    d, f, E = layer.d_model, layer.d_ff, layer.n_experts
    P = T * k
    def workspace(nbytes):
        t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-t.data_ptr()) % 256
        return t[off:off + nbytes]

    ws_bytes = moe_workspace_size(d, f, E, T, k)
    ws_sh_bytes = moe_workspace_size(d, f, E, T, 1)
    z = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=device)
    b = Buffers(T, k, z(max(T, 1), E), z(max(T, 1), k, dt=torch.int32), z(max(T, 1), k),
                z(E + 1, dt=torch.int32), z(max(P, 1), dt=torch.int32), z(max(P, 1), dt=torch.int32),
                z(max(P, 1), d), z(max(T, 1), d), z(max(T, 1), d), workspace(ws_bytes), ws_bytes,
                workspace(ws_sh_bytes), ws_sh_bytes)
    moe_workspace_init(b.ws, b.ws_bytes, stream)
    moe_workspace_init(b.ws_sh, b.ws_sh_bytes, stream)
    return b


class SideStream:
    """A second stream plus the two events of a fork and a join."""

    def __init__(self, device="cuda"):
        self.stream = torch.cuda.Stream(device=device)   # default priority
        self.handle = self.stream.cuda_stream
        self.fork, self.join = hip.Event(), hip.Event()


def run_layer(layer: DeviceLayer, x, b: Buffers, stream=None, logits_in=False, tail_from=None,
              fused=False, side: SideStream | None = None, fuse_combine=False):
    """x: [T][d] bf16 (or int16 bits) device tensor.  Runs route -> dispatch ->
    expert FFN -> combine; returns b.out.  tail_from (< k) switches on route
    tail-skip in the dispatch step; fused uses moe_route_dispatch for the
    first two steps.  With `side` (and an explicit stream handle) the shared
    expert runs on the side stream beside routing and the routed experts
    after it; the streams join before the combine.  fuse_combine uses
    moe_expert_ffn_combine for the last two steps."""
    T, k = b.T, b.k
    d, E = layer.d_model, layer.n_experts
    if side is not None:
        assert stream is not None and not logits_in
        side.fork.record(stream)
        hip.stream_wait_event(side.handle, side.fork)
        moe_shared_ffn(layer.struct, x, T, b.y_shared, b.ws_sh, b.ws_sh_bytes, side.handle)
        side.join.record(side.handle)
    if fused and tail_from is not None:
        assert not logits_in
        moe_route_dispatch_tail_skip(x, layer.router, layer.bias, b.logits, T, d, E, k, tail_from, b.ids,
                                     b.w, b.offsets, b.sorted_pair, b.pair_pos, b.ws, b.ws_bytes, stream)
    elif fused:
        assert not logits_in
        moe_route_dispatch(x, layer.router, layer.bias, b.logits, T, d, E, k, b.ids, b.w, b.offsets,
                           b.sorted_pair, b.pair_pos, b.ws, b.ws_bytes, stream)
    elif logits_in:
        moe_route(None, None, None, b.logits, T, d, E, k, b.ids, b.w, b.ws, b.ws_bytes, stream)
    else:
        moe_route(x, layer.router, layer.bias, b.logits, T, d, E, k, b.ids, b.w, b.ws, b.ws_bytes,
                  stream)
    if fused:
        pass
    elif tail_from is None:
        moe_dispatch(b.ids, T, E, k, b.offsets, b.sorted_pair, b.pair_pos, b.ws, b.ws_bytes, stream)
    else:
        moe_dispatch_tail_skip(b.ids, T, E, k, tail_from, b.offsets, b.sorted_pair, b.pair_pos, b.ws,
                               b.ws_bytes, stream)
    if fuse_combine:
        assert side is None
        moe_expert_ffn_combine(layer.struct, x, T, k, b.offsets, b.sorted_pair, b.pair_pos, b.w, b.y_pairs,
                               b.y_shared, b.out, b.ws, b.ws_bytes, stream)
        return b.out
    if side is not None:
        moe_routed_ffn(layer.struct, x, T, k, b.offsets, b.sorted_pair, b.y_pairs, b.ws, b.ws_bytes,
                       stream)
        hip.stream_wait_event(stream, side.join)
    else:
        moe_expert_ffn(layer.struct, x, T, k, b.offsets, b.sorted_pair, b.y_pairs, b.y_shared, b.ws,
                       b.ws_bytes, stream)
    moe_combine(b.y_pairs, b.y_shared, b.pair_pos, b.w, T, k, d, b.out, stream)
    return b.out
