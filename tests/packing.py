"""Test-side packer: integer codes and fp16 scales -> the library's planes.

This is the forward direction of the storage format declared in
include/moe.h (the oracle implements the reverse, decoding, independently).
Used to build hand-made and adversarial weights for pins and parity tests.

Format, one rows x K matrix (rows % 16 == 0, K % 128 == 0):
  unit u = (r // 16) * (K // 128) + k // 128, rr = r % 16, j = (k % 128) // 32,
  g = (k % 32) // 8, s = k % 8, c = s % 4.
  lo    512 B/unit: byte ((g*16 + rr)*4 + j)*2 + s//4, bits at 4*(c&1) + 2*(c>>1).
  hi    256 B/unit (Q3): little-endian 32-bit word g*16 + rr, bit 4*n + t,
        n = 4*(j%2) + 2*(s//4) + s%2, t = 2*(j//2) + (s//2)%2.
  scale 64 fp16/unit: element rr*4 + j.   min: same (Q2).
"""
import numpy as np


def _positions(rows, K):
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    KC = K // 128
    unit = (r // 16) * KC + k // 128
    rr, j, g, s = r % 16, (k % 128) // 32, (k % 32) // 8, k % 8
    c = s % 4
    lo_byte = unit * 512 + ((g * 16 + rr) * 4 + j) * 2 + s // 4
    lo_shift = 4 * (c & 1) + 2 * (c >> 1)
    hbit = 4 * (4 * (j % 2) + 2 * (s // 4) + s % 2) + 2 * (j // 2) + (s // 2) % 2
    hi_byte = unit * 256 + (g * 16 + rr) * 4 + hbit // 8
    hi_shift = hbit % 8
    sidx = unit * 64 + rr * 4 + j
    return lo_byte, lo_shift, hi_byte, hi_shift, sidx


def pack(codes, scale_f, min_f=None, fmt=1):
    """codes: int [n][rows][K] (0..3 for Q2, 0..7 for Q3);
    scale_f/min_f: float [n][rows][K//32] (rounded to fp16 here).
    Returns dict(lo, hi, scale, min) of flat numpy arrays."""
    codes = np.asarray(codes)
    n, rows, K = codes.shape
    lo_b, lo_s, hi_b, hi_s, sidx = _positions(rows, K)
    nu = (rows // 16) * (K // 128)
    lo = np.zeros(n * nu * 512, np.uint8)
    hi = np.zeros(n * nu * 256, np.uint8) if fmt == 2 else None
    sc = np.zeros(n * nu * 64, np.uint16)
    mn = np.zeros(n * nu * 64, np.uint16) if fmt == 1 else None
    r = np.arange(rows)[:, None]
    kb = np.arange(K // 32)[None, :]
    # block (r, kb) -> scale index, taken at the block's first column
    first = sidx[:, ::32]
    for e in range(n):
        q = codes[e].astype(np.int64)
        np.bitwise_or.at(lo, (e * nu * 512 + lo_b).ravel(), ((q & 3) << lo_s).astype(np.uint8).ravel())
        if fmt == 2:
            np.bitwise_or.at(hi, (e * nu * 256 + hi_b).ravel(), (((q >> 2) & 1) << hi_s).astype(np.uint8).ravel())
        sc[e * nu * 64 + first] = np.asarray(scale_f[e], np.float16).view(np.uint16)[r, kb]
        if fmt == 1:
            mn[e * nu * 64 + first] = np.asarray(min_f[e], np.float16).view(np.uint16)[r, kb]
    return dict(lo=lo, hi=hi, scale=sc, min=mn)


class Mat:
    """Duck-typed matrix set accepted by the oracle wrapper and the GPU binding."""

    def __init__(self, fmt, n, rows, K, planes):
        self.fmt, self.n, self.rows, self.K = fmt, n, rows, K
        self.lo, self.hi, self.scale, self.min = planes["lo"], planes["hi"], planes["scale"], planes["min"]


def dense(codes, scale_f, min_f=None, fmt=1):
    """Dense float64 weights straight from codes and (fp16-rounded) scales."""
    codes = np.asarray(codes, np.float64)
    d = np.repeat(np.asarray(scale_f, np.float16).astype(np.float64), 32, axis=-1)
    if fmt == 1:
        m = np.repeat(np.asarray(min_f, np.float16).astype(np.float64), 32, axis=-1)
        return d * codes + m
    return d * (codes - 4.0)


def random_mat(rng, fmt, n, rows, K, zero=False):
    """Random codes/scales in the workloads' distributions; returns (Mat, dense[n][rows][K])."""
    qmax = 4 if fmt == 1 else 8
    codes = rng.integers(0, qmax, size=(n, rows, K))
    sc = (0.005 + 0.010 * rng.random((n, rows, K // 32))).astype(np.float16)
    mn = (-1.5 * sc.astype(np.float64)).astype(np.float16) if fmt == 1 else None
    if zero:
        sc[:] = 0
        if mn is not None:
            mn[:] = 0
    planes = pack(codes, sc, mn, fmt)
    return Mat(fmt, n, rows, K, planes), dense(codes, sc, mn, fmt)
