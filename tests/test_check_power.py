"""The parity criterion must reject wrong answers (CPU, oracle only).

The GPU parity tests accept an output when max|err| <= tol * RMS(V) and the
relative L2 error is <= 1e-2 (bf16 paths).  Where outputs are small (long
near-uniform rows, decode over 32768 keys) the absolute bound alone is nearly
vacuous, so this file checks, on the oracle's own outputs for inputs drawn as
the workloads draw them, that the combined criterion rejects an all-zero
output, an output with its rows (tokens) shuffled and, for V2, an output with
the pairs of a token permuted.
"""
import numpy as np
import torch

import oracle
from differential_softmax_attention_diffattn_amd import inputs as inp

TOL_BF16 = 2e-2
REL_L2_BF16 = 1e-2


def passes(got, ref, rms_v, tol=TOL_BF16, rel_l2=REL_L2_BF16) -> bool:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return err <= tol * rms_v and rel <= rel_l2


def rms(t) -> float:
    return float(t.double().square().mean().sqrt())


def test_v1_wrong_outputs_fail():
    w = inp.V1_BF16.with_shape(B=1, T=300, H=2)
    x = inp.v1_inputs(w)
    lam = li = oracle.lambda_init(28)
    ref = oracle.v1_forward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, li, w.eps)
    rv = rms(x["v"])
    assert passes(ref, ref, rv)
    assert not passes(np.zeros_like(ref), ref, rv)
    rng = np.random.default_rng(0)
    assert not passes(ref[:, rng.permutation(ref.shape[1])], ref, rv)
    # the two heads exchanged
    assert not passes(ref[:, :, ::-1], ref, rv)
    # a sign error in lambda (z = O1 + lambda O2) is visible too
    wrong = oracle.v1_forward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], -lam, li, w.eps)
    assert not passes(wrong, ref, rv)


def test_v2_wrong_outputs_fail():
    w = inp.V2_PREFILL.with_shape(B=1, T=300, Hq=16, Hkv=2)
    x = inp.v2_inputs(w)
    ref = oracle.v2_forward(x["q"], x["k"], x["v"], x["logit"])
    rv = rms(x["v"])
    assert passes(ref, ref, rv)
    assert not passes(np.zeros_like(ref), ref, rv)
    rng = np.random.default_rng(1)
    assert not passes(ref[:, rng.permutation(ref.shape[1])], ref, rv)
    assert not passes(ref[:, :, ::-1], ref, rv)
    # the odd head added instead of subtracted
    wrong = oracle.v2_forward(x["q"], x["k"], x["v"], -x["logit"])
    assert not passes(wrong, ref, rv)


def test_v2_long_rows_zero_output_fails_on_relative_l2():
    # on long rows the V2 output is ~RMS(V)/sqrt(n): its RMS is already below
    # the absolute bound at 2048 tokens; the relative check still rejects zeros
    w = inp.V2_PREFILL.with_shape(B=1, T=2048, Hq=4, Hkv=2)
    x = inp.v2_inputs(w)
    rows = np.arange(1536, 2048, 37)
    ref = oracle.v2_forward(x["q"], x["k"], x["v"], x["logit"], rows=rows)
    rv = rms(x["v"])
    assert float(np.sqrt(np.mean(ref ** 2))) < TOL_BF16 * rv
    assert not passes(np.zeros_like(ref), ref, rv)


def test_decode_wrong_outputs_fail():
    w = inp.V2_DECODE.with_shape(B=4, S=4096, Hq=16, Hkv=2, d=128)
    x = inp.decode_inputs(w)
    ref = oracle.v2_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"])
    rv = rms(x["v_cache"])
    assert passes(ref, ref, rv)
    # the output's RMS is below the absolute bound: only the relative check
    # separates zeros from the answer
    assert float(np.sqrt(np.mean(ref ** 2))) < TOL_BF16 * rv
    assert not passes(np.zeros_like(ref), ref, rv)
    assert not passes(ref[::-1], ref, rv)
    assert not passes(ref[:, ::-1], ref, rv)


# ---------------------------------------------------------------------------
# V1 backward: the dlambda bounds (tests/dlambda_check.py) must reject
# dlambda = 0 and dlambda = -ref, on the oracle's state and end to end
# ---------------------------------------------------------------------------

import math  # noqa: E402

import pytest  # noqa: E402

import dlambda_check as dlc  # noqa: E402


def _maps_fp16_p(q, k, v, causal):
    """Per-map O of one head with the attention weights rounded to fp16 before
    P.V and the row sum, as the bf16 forward kernel rounds them (a model of its
    rounding, for the end-to-end bound; fp64 otherwise)."""
    T, d = q.shape
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(T)[None, :] > np.arange(T)[:, None], -np.inf, s)
    p = np.exp(s - s.max(-1, keepdims=True)).astype(np.float16).astype(np.float64)
    return (p @ v) / p.sum(-1, keepdims=True)


# the configurations of the GPU backward tests (B, T, H, d, dv, causal, layer, std)
V1_BWD_CONFIGS = [(1, 64, 2, 64, 128, True, 1, None), (2, 37, 2, 64, 128, True, 3, None),
                  (1, 200, 2, 128, 256, True, 12, None), (1, 130, 2, 128, 256, False, 5, 1.0),
                  (2, 97, 1, 64, 128, False, 28, None), (1, 257, 1, 128, 256, True, 7, 1.0),
                  (2, 129, 2, 64, 128, True, 20, 0.5)]


@pytest.mark.parametrize("B,T,H,d,dv,causal,layer,std", V1_BWD_CONFIGS)
def test_v1_dlambda_bounds_reject_zero_and_negated(B, T, H, d, dv, causal, layer, std):
    w = inp.V1_BF16.with_shape(B=B, T=T, H=H, d=d, dv=dv, std=std or 1.0 / math.sqrt(d))
    x = {k: t.double().numpy() for k, t in inp.v1_inputs(w).items()}
    dy = inp.v1_dy(w).double().numpy()
    lam = li = oracle.lambda_init(layer)
    O1, O2, E1, E2 = (np.zeros_like(x["v"]) for _ in range(4))
    for b in range(B):
        for h in range(H):
            O1[b, :, h] = oracle.v2_heads(x["q1"][b, :, h, None], x["k1"][b, :, h, None],
                                          x["v"][b, :, h, None], causal=causal)[:, 0]
            O2[b, :, h] = oracle.v2_heads(x["q2"][b, :, h, None], x["k2"][b, :, h, None],
                                          x["v"][b, :, h, None], causal=causal)[:, 0]
            E1[b, :, h] = _maps_fp16_p(x["q1"][b, :, h], x["k1"][b, :, h], x["v"][b, :, h], causal)
            E2[b, :, h] = _maps_fp16_p(x["q2"][b, :, h], x["k2"][b, :, h], x["v"][b, :, h], causal)
    terms = dlc.dlambda_terms(O1, O2, dy, lam, li, w.eps)
    ref = float(np.sum(terms))
    # oracle state: always decisive; zero and the negated value fail
    bound = dlc.oracle_state_bound(ref, terms)
    assert dlc.decisive(bound, ref)
    assert abs(0.0 - ref) > bound and abs(-ref - ref) > bound
    # end to end, with the forward error of fp16 P: the modelled kernel value
    # passes, and where the bound is decisive zero and -ref fail
    G1, G2 = dlc.dlambda_sensitivity(O1, O2, dy, lam, li, w.eps)
    e2e_bound, sigma = dlc.end_to_end_bound(ref, terms, G1, G2, E1 - O1, E2 - O2)
    modelled = float(np.sum(dlc.dlambda_terms(E1, E2, dy, lam, li, w.eps)))
    assert abs(modelled - ref) <= e2e_bound
    if (T, layer) == (200, 12):
        # the one configuration the GPU tests decide on the oracle state alone
        assert not dlc.decisive(e2e_bound, ref)
    else:
        assert dlc.decisive(e2e_bound, ref)
        assert abs(0.0 - ref) > e2e_bound and abs(-ref - ref) > e2e_bound
