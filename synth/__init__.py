"""Seeded synthetic inputs for the routed, block-quantized MoE layer.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and packs them into the byte sizes
the library's storage format needs; it holds none of the layer's arithmetic
(no dequantisation, no routing, no matmul).  Because every 2-bit and 1-bit
code is drawn uniformly, random bytes are uniformly distributed codes under
any bit order, so the generator does not depend on the tiled code layout.

Every tensor is drawn from its own counter-based Philox stream keyed by
(seed, workload id, layer, tensor id, expert), so any single expert can be
regenerated on its own and always equals the bulk draw.

Workloads (the shapes of the pages' model: 512 routed experts per layer,
top-10 plus one shared expert, 48 layers; MTP verify uses 1+3 tokens per
pass; prefill reads prompts in 8,192-token chunks):

  id  d     f    E    k   T     layers  format  router bias
  0   256   128  16   2   4     1       Q2      none
  1   2048  768  512  10  1     1       Q2      none
  2   2048  768  512  10  4     48      Q3      Zipf s=1.1
  3   2048  768  512  10  8192  1       Q2      none
  4   2048  768  512  10  8192  48      Q3      Zipf s=1.3

Value distributions: x = bf16(N(0,1)) (round to nearest even);
router weights fp32(N(0,1)/sqrt(d)); block scales d = fp16(U(0.005, 0.015));
Q2 block minimum m = fp16(-1.5*d) (stored, not derived by the kernels);
Zipf bias[e] = -s*ln(rank[e]) with rank a seeded permutation of 1..E.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FMT_Q2 = 1
FMT_Q3 = 2

# tensor ids used in stream keys
_T_X, _T_WR, _T_BIAS = 1, 2, 3
_T_MAT = {"gate": 10, "up": 11, "down": 12, "sh_gate": 13, "sh_up": 14, "sh_down": 15}
_P_LO, _P_HI, _P_SCALE = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    d_model: int
    d_ff: int
    n_experts: int
    k: int
    T: int
    layers: int
    fmt: int
    zipf_s: float  # 0.0 = no router bias

    @property
    def P(self) -> int:
        return self.T * self.k


WORKLOADS = {
    0: Workload(0, "tiny-d256-f128-E16-top2-T4-Q2", 256, 128, 16, 2, 4, 1, FMT_Q2, 0.0),
    1: Workload(1, "decode-T1-d2048-f768-E512-top10-Q2", 2048, 768, 512, 10, 1, 1, FMT_Q2, 0.0),
    2: Workload(2, "mtp-verify-T4-48L-d2048-f768-E512-top10-Q3-zipf1.1", 2048, 768, 512, 10, 4, 48, FMT_Q3, 1.1),
    3: Workload(3, "prefill-T8192-d2048-f768-E512-top10-Q2", 2048, 768, 512, 10, 8192, 1, FMT_Q2, 0.0),
    4: Workload(4, "prefill-T8192-48L-d2048-f768-E512-top10-Q3-zipf1.3", 2048, 768, 512, 10, 8192, 48, FMT_Q3, 1.3),
    # the "coder" variant: 256 of the 512 routed experts kept per layer
    5: Workload(5, "coder-decode-T1-d2048-f768-E256-top10-Q2", 2048, 768, 256, 10, 1, 1, FMT_Q2, 0.0),
    6: Workload(6, "coder-prefill-T8192-d2048-f768-E256-top10-Q2", 2048, 768, 256, 10, 8192, 1, FMT_Q2, 0.0),
}


def custom(d_model, d_ff, n_experts, k, T, fmt=FMT_Q2, zipf_s=0.0, layers=1, wid=100, name="custom"):
    """A workload with arbitrary shape (for edge-case and fuzz tests)."""
    return Workload(wid, name, d_model, d_ff, n_experts, k, T, layers, fmt, zipf_s)


def _rng(*key: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(v) & 0xFFFFFFFF for v in key])
    return np.random.Generator(np.random.Philox(key=ss.generate_state(2, dtype=np.uint64)))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return raw bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def fp16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- activations
def gen_x(w: Workload, layer: int = 0, seed: int = 0, T: int | None = None, stream: int = 0) -> np.ndarray:
    """x as bf16 bits, shape [T][d_model]."""
    T = w.T if T is None else T
    g = _rng(seed, w.wid, layer, _T_X, stream)
    v = g.standard_normal((T, w.d_model)).astype(np.float32)
    return _f32_to_bf16_bits(v)


def gen_router(w: Workload, layer: int = 0, seed: int = 0) -> np.ndarray:
    """Router weights fp32, shape [d_model][E] (E contiguous)."""
    g = _rng(seed, w.wid, layer, _T_WR, 0)
    v = g.standard_normal((w.d_model, w.n_experts)) / math.sqrt(w.d_model)
    return v.astype(np.float32)


def gen_bias(w: Workload, layer: int = 0, seed: int = 0) -> np.ndarray | None:
    """Per-expert Zipf(s) router bias: -s*ln(rank[e]); None when s == 0."""
    if w.zipf_s == 0.0:
        return None
    g = _rng(seed, w.wid, layer, _T_BIAS, 0)
    rank = g.permutation(w.n_experts) + 1
    return (-w.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


# ---------------------------------------------------------------- quantized weights
def plane_sizes(fmt: int, rows: int, K: int) -> dict:
    """Bytes (lo, hi) and element counts (scale, min) of one rows x K matrix."""
    nblk = rows * K // 32
    return {
        "lo": rows * K // 4,
        "hi": rows * K // 8 if fmt == FMT_Q3 else 0,
        "scale": nblk,
        "min": nblk if fmt == FMT_Q2 else 0,
    }


def _gen_one(fmt, rows, K, seed, wid, layer, tid, expert):
    s = plane_sizes(fmt, rows, K)
    lo = np.frombuffer(_rng(seed, wid, layer, tid, _P_LO, expert).bytes(s["lo"]), dtype=np.uint8)
    hi = None
    if s["hi"]:
        hi = np.frombuffer(_rng(seed, wid, layer, tid, _P_HI, expert).bytes(s["hi"]), dtype=np.uint8)
    u = _rng(seed, wid, layer, tid, _P_SCALE, expert).random(s["scale"])
    dsc = (0.005 + 0.010 * u).astype(np.float16)  # float64 -> fp16, nearest-even
    mn = None
    if s["min"]:
        mn = (-1.5 * dsc.astype(np.float64)).astype(np.float16)
    return lo, hi, dsc.view(np.uint16), (mn.view(np.uint16) if mn is not None else None)


@dataclasses.dataclass
class QMat:
    """n stacked rows x K matrices in the library's packed planes (host copy)."""
    fmt: int
    n: int
    rows: int
    K: int
    lo: np.ndarray      # uint8  [n * rows*K/4]
    hi: np.ndarray | None     # uint8  [n * rows*K/8]      (Q3)
    scale: np.ndarray   # uint16 [n * rows*K/32]     (fp16 bits)
    min: np.ndarray | None    # uint16 [n * rows*K/32]     (Q2, fp16 bits)

    def expert(self, e: int) -> "QMat":
        s = plane_sizes(self.fmt, self.rows, self.K)
        sl = lambda a, sz: None if a is None else a[e * sz:(e + 1) * sz]
        return QMat(self.fmt, 1, self.rows, self.K, sl(self.lo, s["lo"]), sl(self.hi, s["hi"]),
                    sl(self.scale, s["scale"]), sl(self.min, s["min"]))


def gen_qmat(w: Workload, which: str, layer: int = 0, seed: int = 0, experts=None) -> QMat:
    """One of gate/up/down (routed, n = E) or sh_gate/sh_up/sh_down (n = 1).

    gate/up: rows = d_ff, K = d_model.  down: rows = d_model, K = d_ff.
    `experts` restricts generation to a list of expert indices (stacked in that order).
    """
    tid = _T_MAT[which]
    rows, K = (w.d_model, w.d_ff) if which.endswith("down") else (w.d_ff, w.d_model)
    n_all = 1 if which.startswith("sh_") else w.n_experts
    ids = list(range(n_all)) if experts is None else list(experts)
    parts = [_gen_one(w.fmt, rows, K, seed, w.wid, layer, tid, e) for e in ids]
    cat = lambda i: None if parts[0][i] is None else np.concatenate([p[i] for p in parts])
    return QMat(w.fmt, len(ids), rows, K, cat(0), cat(1), cat(2), cat(3))


@dataclasses.dataclass
class Layer:
    w: Workload
    gate: QMat
    up: QMat
    down: QMat
    sh_gate: QMat
    sh_up: QMat
    sh_down: QMat
    router: np.ndarray
    bias: np.ndarray | None


def gen_layer(w: Workload, layer: int = 0, seed: int = 0) -> Layer:
    return Layer(w,
                 gen_qmat(w, "gate", layer, seed), gen_qmat(w, "up", layer, seed),
                 gen_qmat(w, "down", layer, seed), gen_qmat(w, "sh_gate", layer, seed),
                 gen_qmat(w, "sh_up", layer, seed), gen_qmat(w, "sh_down", layer, seed),
                 gen_router(w, layer, seed), gen_bias(w, layer, seed))
