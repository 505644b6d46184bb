"""GPU: inputs far from unit scale, on the decode (T <= 16) and the prefill
(T > 16) paths.

Both paths stage activations in fp16 (prefill: x and h; decode: h), whose
range ends at 65504.  Each token row is scaled by an exact power of two
before that rounding (undone in fp32 afterwards), so x scaled by 2^8 .. 2^12
(h then reaches ~10^6 .. 10^9) or by 2^-20 .. 2^-40 gives the same relative
accuracy as unit-scale x.  Checked per token against the oracle (routing on
the GPU's own logits), and decode against prefill on the same tokens.
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


@pytest.fixture(scope="module")
def layers():
    """(workload, host layer, device layer) for Q2 and Q3 at the real shape."""
    from quantized_moe_route_amd.layer import DeviceLayer
    out = {}
    for fmt, wid in ((1, 1), (2, 2)):
        w = synth.WORKLOADS[wid]
        L = synth.gen_layer(w)
        out[fmt] = (w, L, DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L, L.router, L.bias))
    return out


def _scaled_x(w, T, exps, seed):
    """bf16 bits of N(0,1) rows, token t multiplied by 2^exps[t % len] (exact)."""
    x = synth.bf16_bits_to_f32(synth.gen_x(w, T=T, seed=seed)).astype(np.float64)
    sc = np.array([2.0 ** exps[t % len(exps)] for t in range(T)])
    xs = (x * sc[:, None]).astype(np.float32)
    bits = (xs.view(np.uint32) >> 16).astype(np.uint16)   # exact: x is bf16 and 2^e is a power of two
    assert np.array_equal(synth.bf16_bits_to_f32(bits), xs)
    return bits


def _run(q, dl, w, x_bits):
    from quantized_moe_route_amd.layer import alloc_buffers, run_layer
    T = x_bits.shape[0]
    b = alloc_buffers(dl, T, w.k)
    run_layer(dl, torch.from_numpy(x_bits.view(np.int16)).cuda(), b)
    torch.cuda.synchronize()
    return b.logits[:T].cpu().numpy(), b.ids[:T].cpu().numpy(), b.out[:T].cpu().numpy()


def _per_token_err(out, ref):
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    return np.max(np.abs(np.asarray(out, np.float64) - ref), axis=1) / rms


CASES = [
    # (T, exponents cycled over the tokens)
    (1, [8]), (1, [10]), (1, [12]), (1, [-20]), (1, [-40]),
    (4, [12, 0, -30, 8]),
    (16, [12, 8, 0, -20, -40, 10]),
    (64, [12, 8, 0, -20, -40, 10]),
    (300, [12, -40, 0, 9]),
]


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("T,exps", CASES)
def test_scaled_inputs_match_oracle(q, layers, fmt, T, exps):
    w, L, dl = layers[fmt]
    x = _scaled_x(w, T, exps, seed=T + 31 * fmt)
    print(f"fmt {fmt} T {T} exponents {exps}", flush=True)
    lg, ids, out = _run(q, dl, w, x)
    assert np.all(np.isfinite(out))
    ids_ref, _ = oracle.topk_softmax(lg, w.k)
    assert np.array_equal(ids, ids_ref)
    _, _, ref = oracle.layer(L, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x, logits=lg)
    err = _per_token_err(out, ref)
    print(f"worst token max|err|/rms = {err.max():.3e}")
    assert err.max() <= TOL


@pytest.mark.parametrize("fmt", [1, 2])
def test_decode_and_prefill_paths_agree(q, layers, fmt):
    """The same 16 scaled tokens through the decode path (T = 16) and, with
    one more token, the prefill path (T = 17): per token within tolerance."""
    w, L, dl = layers[fmt]
    x = _scaled_x(w, 17, [12, 8, 0, -20, -40, 10, 4], seed=700 + fmt)
    _, _, out_dec = _run(q, dl, w, x[:16])
    _, _, out_pre = _run(q, dl, w, x)
    err = _per_token_err(out_dec, out_pre[:16])
    print(f"decode vs prefill: worst token max|diff|/rms = {err.max():.3e}")
    assert err.max() <= 2 * TOL
