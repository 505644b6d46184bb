"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a brute force, a library routine, a
closed form, an invariant or a hand-derived fixture, chosen so that a
plausible slip in the oracle (a dropped term, a swapped bit, a wrong index or
sign, a transposed operand) fails at least one of them.  CPU only.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import packing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ numbers
def test_fp16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(int(b)) for b in bits[::7]])
    r = ref[::7]
    finite = np.isfinite(r)
    assert np.array_equal(got[finite], r[finite])
    assert np.all(np.isnan(got[np.isnan(r)]))
    assert np.array_equal(got[np.isinf(r)], r[np.isinf(r)])


def test_bf16_decode_matches_float32_view():
    bits = np.arange(0, 65536, 13, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


# ------------------------------------------------------------------ dequant
def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].split()
            if line:
                rows.append(line)
    return rows


def test_q2_golden_unit_bytes_and_values():
    fx = _read_fixture("q2_unit.txt")
    codes = np.zeros((1, 16, 128), np.int64)
    for kind, *v in fx:
        if kind == "code":
            codes[0, int(v[0]), int(v[1])] = int(v[2])
    lo = np.zeros(512, np.uint8)
    for kind, *v in fx:
        if kind == "byte":
            lo[int(v[0])] = int(v[1], 16)
    m = packing.Mat(1, 1, 16, 128, dict(lo=lo, hi=None,
                                        scale=np.full(64, 0x3C00, np.uint16),
                                        min=np.full(64, 0xBE00, np.uint16)))
    table = {0: -1.5, 1: -0.5, 2: 0.5, 3: 1.5}
    dq = oracle.dequant_matrix(m, 1, 16, 128)
    for r in range(16):
        for k in range(128):
            assert oracle.code(m, 1, 16, 128, 0, r, k) == codes[0, r, k], (r, k)
            assert dq[r, k] == table[int(codes[0, r, k])]
    # the test-side packer produces the same bytes from the same codes
    p = packing.pack(codes, np.ones((1, 16, 4)), np.full((1, 16, 4), -1.5), fmt=1)
    assert np.array_equal(p["lo"], lo)


def test_q3_golden_unit_bytes_and_values():
    fx = _read_fixture("q3_unit.txt")
    codes = np.zeros((1, 16, 128), np.int64)
    lo = np.zeros(512, np.uint8)
    hi = np.zeros(256, np.uint8)
    for kind, *v in fx:
        if kind == "code":
            codes[0, int(v[0]), int(v[1])] = int(v[2])
        elif kind == "lo":
            lo[int(v[0])] = int(v[1], 16)
        elif kind == "hi":
            hi[int(v[0])] = int(v[1], 16)
    m = packing.Mat(2, 1, 16, 128, dict(lo=lo, hi=hi, scale=np.full(64, 0x3800, np.uint16), min=None))
    dq = oracle.dequant_matrix(m, 2, 16, 128)
    table = {q: 0.5 * (q - 4) for q in range(8)}
    for r in range(16):
        for k in range(128):
            assert oracle.code(m, 2, 16, 128, 0, r, k) == codes[0, r, k], (r, k)
            assert dq[r, k] == table[int(codes[0, r, k])]
    p = packing.pack(codes, np.full((1, 16, 4), 0.5), None, fmt=2)
    assert np.array_equal(p["lo"], lo) and np.array_equal(p["hi"], hi)


@pytest.mark.parametrize("fmt", [1, 2])
def test_single_code_at_every_bit_position(fmt):
    """One non-zero code at a time, at every column of a 16x128 unit and a few
    rows: the oracle must find it exactly there and nowhere else."""
    qmax = 3 if fmt == 1 else 7
    for r in (0, 7, 15):
        for k in range(128):
            codes = np.zeros((1, 16, 128), np.int64)
            codes[0, r, k] = qmax
            sc = np.ones((1, 16, 4))
            mn = np.zeros((1, 16, 4)) if fmt == 1 else None
            m = packing.Mat(fmt, 1, 16, 128, packing.pack(codes, sc, mn, fmt))
            got = np.array([[oracle.code(m, fmt, 16, 128, 0, rr, kk) for kk in range(128)] for rr in range(16)])
            assert np.array_equal(got, codes[0]), (r, k)


@pytest.mark.parametrize("fmt", [1, 2])
def test_dequant_roundtrip_random(fmt):
    rng = np.random.default_rng(5)
    m, dense = packing.random_mat(rng, fmt, 3, 32, 256)
    for e in range(3):
        assert np.array_equal(oracle.dequant_matrix(m, fmt, 32, 256, e), dense[e])


def test_fp32_dequant_is_exact_for_generator_scales():
    """d*q + m (Q2) and d*(q-4) (Q3) are exact in fp32 for every fp16 d in
    [0.005, 0.015] with m = fp16(-1.5 d): brute force over all such d."""
    lo = np.float16(0.005).view(np.uint16)
    hi = np.float16(0.015).view(np.uint16)
    d16 = np.arange(lo, hi + 1, dtype=np.uint16).view(np.float16)
    d = d16.astype(np.float64)
    m = (-1.5 * d).astype(np.float16).astype(np.float64)
    for q in range(4):
        exact = d * q + m
        f32 = (d.astype(np.float32) * np.float32(q) + m.astype(np.float32)).astype(np.float64)
        assert np.array_equal(exact, f32)
    for q in range(8):
        exact = d * (q - 4)
        f32 = (d.astype(np.float32) * np.float32(q - 4)).astype(np.float64)
        assert np.array_equal(exact, f32)


# ------------------------------------------------------------------ routing
def test_router_logits_vs_numpy_matmul():
    w = synth.WORKLOADS[0]
    x = synth.gen_x(w)
    wr = synth.gen_router(w)
    got = oracle.router_logits(x, wr)
    ref = (synth.bf16_bits_to_f32(x).astype(np.float64) @ wr.astype(np.float64)).astype(np.float32)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    bias = np.linspace(-2, 1, w.n_experts).astype(np.float32)
    gb = oracle.router_logits(x, wr, bias)
    assert np.array_equal(gb, got + bias[None, :])


def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(16, 2), (512, 10), (64, 64), (7, 1)])
def test_topk_vs_brute_force_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    T = 40
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:10] = np.round(lg[:10] * 2)          # many exact ties
    lg[10:12] = 0.0
    lg[10, ::3] = -0.0                       # signed zeros tie with +0.0
    lg[12] = 5.0                             # all equal
    ids, w = oracle.topk_softmax(lg, k)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(lg[t], k), t


def test_topk_weights_closed_forms():
    rng = np.random.default_rng(1)
    T, E, k = 64, 512, 10
    lg = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    ids, w = oracle.topk_softmax(lg, k)
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    # softmax over all E restricted to the top-k and renormalised equals the
    # softmax of the k selected logits alone
    sel = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.max(np.abs(w - ref)) < 1e-7
    ids1, w1 = oracle.topk_softmax(lg, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], np.argmax(lg, 1))


# ----------------------------------------------------------------- dispatch
@pytest.mark.parametrize("T,E,k", [(4, 16, 2), (1, 512, 10), (300, 64, 8), (50, 1, 1), (33, 512, 10)])
def test_dispatch_invariants_and_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, sp, pp = oracle.dispatch(ids, E)
    P = T * k
    flat = ids.ravel()
    assert off[0] == 0 and off[E] == P and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))
    assert np.array_equal(pp[sp], np.arange(P))
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_dispatch_skewed_and_empty_experts():
    T, E, k = 200, 32, 4
    ids = np.tile(np.array([3, 7, 0, 31], np.int32), (T, 1))
    off, sp, pp = oracle.dispatch(ids, E)
    sizes = np.diff(off)
    assert sizes[3] == T and sizes[7] == T and sizes[0] == T and sizes[31] == T
    assert sizes.sum() == T * k and np.count_nonzero(sizes) == 4
    assert np.array_equal(sp, np.argsort(ids.ravel(), kind="stable"))


# ------------------------------------------------------------------- experts
def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dense_ffn(x, Wg, Wu, Wd):
    return (_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T


def _make_layer(rng, fmt, d, f, E, zero_routed=False, same=False):
    g, Dg = packing.random_mat(rng, fmt, E, f, d, zero=zero_routed)
    u, Du = packing.random_mat(rng, fmt, E, f, d, zero=zero_routed)
    dn, Dd = packing.random_mat(rng, fmt, E, d, f, zero=zero_routed)
    if same:  # every routed expert gets expert 0's weights
        for mat in (g, u, dn):
            for name in ("lo", "hi", "scale", "min"):
                a = getattr(mat, name)
                if a is not None:
                    per = a.size // E
                    a[:] = np.tile(a[:per], E)
        Dg, Du, Dd = (np.repeat(D[:1], E, 0) for D in (Dg, Du, Dd))
    sg, Dsg = packing.random_mat(rng, fmt, 1, f, d)
    su, Dsu = packing.random_mat(rng, fmt, 1, f, d)
    sd, Dsd = packing.random_mat(rng, fmt, 1, d, f)

    class L:
        pass

    L.gate, L.up, L.down, L.sh_gate, L.sh_up, L.sh_down = g, u, dn, sg, su, sd
    dense = dict(g=Dg, u=Du, d=Dd, sg=Dsg[0], su=Dsu[0], sd=Dsd[0])
    return L, dense


def _x(rng, T, d):
    return synth._f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))


@pytest.mark.parametrize("fmt", [1, 2])
def test_single_expert_equals_dense_swiglu(fmt):
    """E = 1, k = 1: weight 1, out = FFN_0(x) + FFN_shared(x) by numpy float64."""
    rng = np.random.default_rng(10 + fmt)
    d, f, T = 256, 128, 5
    L, D = _make_layer(rng, fmt, d, f, 1)
    x = _x(rng, T, d)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wr = rng.standard_normal((d, 1)).astype(np.float32)
    ids, w, out = oracle.layer(L, fmt, d, f, 1, 1, x, wr=wr)
    assert np.all(ids == 0) and np.all(w == 1.0)
    ref = _dense_ffn(xf, D["g"][0], D["u"][0], D["d"][0]) + _dense_ffn(xf, D["sg"], D["su"], D["sd"])
    assert np.max(np.abs(out - ref)) <= 1e-6 * np.max(np.abs(ref))


@pytest.mark.parametrize("fmt", [1, 2])
def test_expert_rows_h_and_y_vs_numpy(fmt):
    rng = np.random.default_rng(20 + fmt)
    d, f, E = 256, 128, 4
    L, D = _make_layer(rng, fmt, d, f, E)
    x = _x(rng, 3, d)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    re = np.array([2, -1, 0, 3], np.int32)
    rt = np.array([0, 1, 2, 2], np.int32)
    y, h = oracle.expert_rows(L, fmt, d, f, E, x, re, rt, want_h=True, f64=True)
    for i in range(4):
        if re[i] < 0:
            Wg, Wu, Wd = D["sg"], D["su"], D["sd"]
        else:
            Wg, Wu, Wd = D["g"][re[i]], D["u"][re[i]], D["d"][re[i]]
        hh = _silu(xf[rt[i]] @ Wg.T) * (xf[rt[i]] @ Wu.T)
        assert np.allclose(h[i], hh, rtol=1e-12, atol=1e-14)
        assert np.allclose(y[i], hh @ Wd.T, rtol=1e-12, atol=1e-14)


def test_identical_experts_make_output_independent_of_routing():
    rng = np.random.default_rng(33)
    d, f, E, k, T = 128, 128, 8, 3, 4
    L, D = _make_layer(rng, 1, d, f, E, same=True)
    x = _x(rng, T, d)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    lg1 = rng.standard_normal((T, E)).astype(np.float32)
    lg2 = rng.standard_normal((T, E)).astype(np.float32)
    _, _, o1 = oracle.layer(L, 1, d, f, E, k, x, logits=lg1)
    i2, _, o2 = oracle.layer(L, 1, d, f, E, k, x, logits=lg2)
    ref = _dense_ffn(xf, D["g"][0], D["u"][0], D["d"][0]) + _dense_ffn(xf, D["sg"], D["su"], D["sd"])
    tol = 1e-6 * np.max(np.abs(ref))
    assert np.max(np.abs(o1 - ref)) <= tol and np.max(np.abs(o2 - ref)) <= tol


def test_token_independence_batch_equals_single_tokens():
    w = synth.WORKLOADS[0]
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    ids, wt, out = oracle.layer(L, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x, wr=L.router)
    for t in range(w.T):
        i1, w1, o1 = oracle.layer(L, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x[t:t + 1], wr=L.router)
        assert np.array_equal(i1[0], ids[t]) and np.array_equal(w1[0], wt[t])
        assert np.array_equal(o1[0], out[t])


def test_zero_routed_weights_leave_shared_expert():
    rng = np.random.default_rng(44)
    d, f, E, k, T = 128, 128, 8, 2, 3
    L, D = _make_layer(rng, 1, d, f, E, zero_routed=True)
    x = _x(rng, T, d)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    _, _, out = oracle.layer(L, 1, d, f, E, k, x, logits=rng.standard_normal((T, E)).astype(np.float32))
    ref = _dense_ffn(xf, D["sg"], D["su"], D["sd"])
    assert np.max(np.abs(out - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_relabelling_experts_permutes_ids_only():
    rng = np.random.default_rng(55)
    d, f, E, k, T = 128, 128, 8, 3, 6
    L, _ = _make_layer(rng, 1, d, f, E)
    x = _x(rng, T, d)
    wr = rng.standard_normal((d, E)).astype(np.float32)
    ids, w, out = oracle.layer(L, 1, d, f, E, k, x, wr=wr)
    perm = rng.permutation(E)              # new label e' holds old expert perm[e']
    L2, _ = _make_layer(rng, 1, d, f, E)
    for name in ("gate", "up", "down"):
        src, dst = getattr(L, name), getattr(L2, name)
        for pl in ("lo", "hi", "scale", "min"):
            a = getattr(src, pl)
            if a is None:
                continue
            per = a.size // E
            b = np.concatenate([a[perm[e] * per:(perm[e] + 1) * per] for e in range(E)])
            getattr(dst, pl)[:] = b
    for name in ("sh_gate", "sh_up", "sh_down"):
        setattr(L2, name, getattr(L, name))
    ids2, w2, out2 = oracle.layer(L2, 1, d, f, E, k, x, wr=wr[:, perm])
    inv = np.argsort(perm)
    assert np.array_equal(ids2, inv[ids]) and np.array_equal(w2, w)
    assert np.array_equal(out2, out)


def test_down_scale_power_of_two_scales_routed_output_exactly():
    rng = np.random.default_rng(66)
    d, f, E = 128, 128, 3
    L, _ = _make_layer(rng, 1, d, f, E)
    x = _x(rng, 2, d)
    re = np.array([0, 1, 2, 1], np.int32)
    rt = np.array([0, 0, 1, 1], np.int32)
    y1 = oracle.expert_rows(L, 1, d, f, E, x, re, rt, f64=True)
    for pl in ("scale", "min"):
        a = getattr(L.down, pl)
        a[:] = (a.view(np.float16).astype(np.float64) * 2.0).astype(np.float16).view(np.uint16)
    y2 = oracle.expert_rows(L, 1, d, f, E, x, re, rt, f64=True)
    assert np.array_equal(y2, 2.0 * y1)


def test_combine_vs_numpy():
    rng = np.random.default_rng(77)
    T, k, d = 9, 4, 64
    P = T * k
    yp = rng.standard_normal((P, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32)
    pp = rng.permutation(P).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.combine(yp, ys, pp, w, T, k, d)
    ref = ys.astype(np.float64) + np.einsum("tj,tjd->td", w.astype(np.float64),
                                            yp[pp.reshape(T, k)].astype(np.float64))
    assert np.max(np.abs(out - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_layer_equals_composition_of_steps():
    """oracle.layer == router -> topk -> dispatch -> expert rows -> combine."""
    w = synth.WORKLOADS[0]
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    ids, wt, out = oracle.layer(L, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x, wr=L.router)
    lg = oracle.router_logits(x, L.router)
    ids2, w2 = oracle.topk_softmax(lg, w.k)
    off, sp, pp = oracle.dispatch(ids2, w.n_experts)
    flat = ids2.ravel()
    re = np.concatenate([flat[sp], -np.ones(w.T, np.int32)])
    rt = np.concatenate([sp // w.k, np.arange(w.T)]).astype(np.int32)
    y = oracle.expert_rows(L, w.fmt, w.d_model, w.d_ff, w.n_experts, x, re, rt)
    out2 = oracle.combine(y[:w.P], y[w.P:], pp, w2, w.T, w.k, w.d_model)
    assert np.array_equal(ids, ids2) and np.array_equal(wt, w2)
    assert np.max(np.abs(out - out2)) <= 1e-6 * np.sqrt(np.mean(out.astype(np.float64) ** 2))


# ------------------------------------------------------------ route tail-skip
def _read_int_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].split()
            if line:
                vals[line[0]] = [int(v) for v in line[1:]]
    return vals


def test_tail_skip_hand_example():
    g = _read_int_fixture("tail_skip_example.txt")
    T, k, E, tf = g["T"][0], g["k"][0], g["E"][0], g["tail_from"][0]
    ids = np.array(g["ids"], np.int32).reshape(T, k)
    assert np.array_equal(oracle.tail_keep(ids, E, tf), np.array(g["keep"], bool))
    off, sp, pp = oracle.dispatch_tail_skip(ids, E, tf)
    n = off[E]
    assert np.array_equal(off, g["offsets"])
    assert np.array_equal(sp[:n], g["sorted_pair"])
    assert np.array_equal(pp, g["pair_pos"])


def _tail_skip_brute(ids, E, tf):
    """Loops straight from the rule: keep e iff some (t, j < tf) picks e."""
    T, k = ids.shape
    keep = [False] * E
    for t in range(T):
        for j in range(min(tf, k)):
            keep[ids[t, j]] = True
    offsets, sp, pp = [], [], [-1] * (T * k)
    for e in range(E):
        offsets.append(len(sp))
        for p in range(T * k):
            if ids[p // k, p % k] == e and keep[e]:
                pp[p] = len(sp)
                sp.append(p)
    offsets.append(len(sp))
    return np.array(keep), np.array(offsets), np.array(sp, np.int64), np.array(pp)


@pytest.mark.parametrize("seed", range(12))
def test_tail_skip_vs_brute_force(seed):
    rng = np.random.default_rng(900 + seed)
    T, E = int(rng.integers(1, 20)), int(rng.integers(2, 13))
    k = int(rng.integers(1, min(E, 6) + 1))
    tf = int(rng.integers(0, k + 1))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    keep, off_b, sp_b, pp_b = _tail_skip_brute(ids, E, tf)
    off, sp, pp = oracle.dispatch_tail_skip(ids, E, tf)
    assert np.array_equal(oracle.tail_keep(ids, E, tf), keep)
    assert np.array_equal(off, off_b)
    assert np.array_equal(sp[:off[E]], sp_b)
    assert np.array_equal(pp, pp_b)


def test_tail_skip_special_cases():
    rng = np.random.default_rng(31)
    E, k = 512, 10
    # one token: exactly its first tail_from picks survive, in expert order
    ids1 = rng.permutation(E)[:k].astype(np.int32)[None, :]
    off, sp, pp = oracle.dispatch_tail_skip(ids1, E, 6)
    assert off[E] == 6 and np.all(pp[6:] == -1)
    assert np.array_equal(sp[:6], np.argsort(ids1[0, :6], kind="stable"))
    # tail_from = k: the plain dispatch, bit for bit
    ids = np.stack([rng.permutation(E)[:k] for _ in range(40)]).astype(np.int32)
    for a, b in zip(oracle.dispatch_tail_skip(ids, E, k), oracle.dispatch(ids, E)):
        assert np.array_equal(a[:len(b)], b)
    # tail_from = 0: nothing is computed
    off, _, pp = oracle.dispatch_tail_skip(ids, E, 0)
    assert np.all(off == 0) and np.all(pp == -1)


def test_layer_tail_skip_equals_composition():
    """oracle.layer(tail_from) == shared + the kept pairs' weighted rows; with
    tail_from = k it is the plain layer; tail_from = 0 leaves the shared
    expert alone."""
    w = synth.custom(128, 128, 24, 6, 5, fmt=2, zipf_s=1.1, wid=930)
    L = synth.gen_layer(w)
    x = synth.gen_x(w)
    d, f, E, k, T = w.d_model, w.d_ff, w.n_experts, w.k, w.T
    lg = oracle.router_logits(x, L.router, L.bias)
    ids, wt = oracle.topk_softmax(lg, k)
    tf = 3
    off, sp, pp = oracle.dispatch_tail_skip(ids, E, tf)
    n = off[E]
    assert 0 < n < T * k
    flat = ids.ravel()
    re = np.concatenate([flat[sp[:n]], -np.ones(T, np.int32)]).astype(np.int32)
    rt = np.concatenate([sp[:n] // k, np.arange(T)]).astype(np.int32)
    y = oracle.expert_rows(L, w.fmt, d, f, E, x, re, rt)
    yp = np.zeros((T * k, d), np.float32)
    yp[:n] = y[:n]
    out_c = oracle.combine(yp, y[n:], pp, wt, T, k, d)
    _, _, out = oracle.layer(L, w.fmt, d, f, E, k, x, logits=lg, tail_from=tf)
    rms = np.sqrt(np.mean(out.astype(np.float64) ** 2))
    assert np.max(np.abs(out - out_c)) <= 1e-6 * rms
    _, _, plain = oracle.layer(L, w.fmt, d, f, E, k, x, logits=lg)
    _, _, same = oracle.layer(L, w.fmt, d, f, E, k, x, logits=lg, tail_from=k)
    assert np.array_equal(plain, same)
    assert np.max(np.abs(out - plain)) > 0.0
    _, _, sh = oracle.layer(L, w.fmt, d, f, E, k, x, logits=lg, tail_from=0)
    ysh = oracle.expert_rows(L, w.fmt, d, f, E, x, -np.ones(T, np.int32), np.arange(T, dtype=np.int32))
    assert np.max(np.abs(sh - ysh)) <= 1e-6 * np.sqrt(np.mean(ysh.astype(np.float64) ** 2))
