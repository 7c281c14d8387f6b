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
