"""Seeded synthetic layers generated directly in GPU memory (torch's Philox).

Same shapes and value distributions as the host generator in this package
(uniform random code bytes, d = fp16(U(0.005, 0.015)), Q2 m = fp16(-1.5 d),
x = bf16(N(0,1)), Wr = N(0,1)/sqrt(d), Zipf bias = -s ln(rank)), but a
different random stream; used where tens of GB of weights (48-layer stacks)
must be resident without a host round trip.  Holds no layer arithmetic.
"""
from __future__ import annotations

import math

import torch

from . import FMT_Q2, FMT_Q3, Workload, plane_sizes

_MATS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")


def _gen(seed: int, *key: int, device="cuda") -> torch.Generator:
    g = torch.Generator(device=device)
    h = seed
    for v in key:
        h = (h * 1000003 + int(v) + 0x9E3779B9) & 0x7FFFFFFFFFFFFFFF
    g.manual_seed(h)
    return g


def layer_planes(w: Workload, layer: int, seed: int = 0, device="cuda") -> dict:
    """name -> (lo uint8, hi uint8|None, scale int16 fp16-bits, min int16|None)."""
    out = {}
    for mi, name in enumerate(_MATS):
        rows, K = (w.d_model, w.d_ff) if name.endswith("down") else (w.d_ff, w.d_model)
        n = 1 if name.startswith("sh_") else w.n_experts
        s = plane_sizes(w.fmt, rows, K)
        g = _gen(seed, w.wid, layer, mi, device=device)
        lo = torch.randint(0, 256, (n * s["lo"],), dtype=torch.uint8, device=device, generator=g)
        hi = (torch.randint(0, 256, (n * s["hi"],), dtype=torch.uint8, device=device, generator=g)
              if w.fmt == FMT_Q3 else None)
        u = torch.rand(n * s["scale"], dtype=torch.float32, device=device, generator=g)
        dsc = (0.005 + 0.010 * u).to(torch.float16)
        mn = (-1.5 * dsc.float()).to(torch.float16) if w.fmt == FMT_Q2 else None
        out[name] = (lo, hi, dsc.view(torch.int16), None if mn is None else mn.view(torch.int16))
        del u
    return out


def router(w: Workload, layer: int, seed: int = 0, device="cuda"):
    g = _gen(seed, w.wid, layer, 100, device=device)
    wr = torch.randn(w.d_model, w.n_experts, dtype=torch.float32, device=device, generator=g)
    wr /= math.sqrt(w.d_model)
    bias = None
    if w.zipf_s:
        rank = torch.randperm(w.n_experts, device=device, generator=g).to(torch.float64) + 1.0
        bias = (-w.zipf_s * torch.log(rank)).to(torch.float32)
    return wr, bias


def x(w: Workload, layer: int, step: int, seed: int = 0, T: int | None = None, device="cuda"):
    """bf16 activations [T][d] as int16 bits."""
    T = w.T if T is None else T
    g = _gen(seed, w.wid, layer, 200 + step, device=device)
    v = torch.randn(T, w.d_model, dtype=torch.float32, device=device, generator=g)
    return v.to(torch.bfloat16).view(torch.int16)


def to_host(planes: dict):
    """Host copy (numpy) of device planes, shaped like the host generator's layer."""
    import numpy as np

    class H:
        pass

    h = H()
    for name, (lo, hi, sc, mn) in planes.items():
        m = H()
        m.lo = lo.cpu().numpy()
        m.hi = None if hi is None else hi.cpu().numpy()
        m.scale = sc.cpu().numpy().view(np.uint16)
        m.min = None if mn is None else mn.cpu().numpy().view(np.uint16)
        setattr(h, name, m)
    return h
