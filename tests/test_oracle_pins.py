"""Pins for the fp64 oracle: each test checks it against something other than itself.

The pins come from what the pages and the mathematics fix: the lambda_init
schedule, the figure 90.5 printed for uniform attention at length 8192, the
reduction to ordinary softmax attention (checked against torch's
scaled_dot_product_attention in float64, an independent library routine),
exact zeros for identical streams, closed forms for uniform and one-hot
attention, structural properties (causality, shift invariance, no leakage
across packed sequences), and scalar brute force on tiny inputs.  Each pin is
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign,
index or axis, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def rng(seed):
    return np.random.default_rng(seed)


def sdpa(q, k, v, causal, gqa=False):
    """torch SDPA in float64 on [T, H, d] arrays (one sequence) -> [T, H, dv]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1)))[None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, enable_gqa=gqa)
    return np.swapaxes(o[0].numpy(), 0, 1)


# ---------------------------------------------------------------------------
# lambda_init
# ---------------------------------------------------------------------------

def test_lambda_init_first_layer_is_page_value():
    assert oracle.lambda_init(1) == pytest.approx(GOLDEN["lambda_init_layer1"]["value"], abs=1e-15)


def test_lambda_init_grows_geometrically_to_limit():
    lim = GOLDEN["lambda_init_limit"]["value"]
    vals = [oracle.lambda_init(l) for l in range(1, 31)]
    assert all(b > a for a, b in zip(vals, vals[1:])), "must grow with depth"
    assert all(v < lim for v in vals)
    # the gap to the limit shrinks by the same factor every layer
    ratios = [(lim - b) / (lim - a) for a, b in zip(vals, vals[1:])]
    assert max(ratios) - min(ratios) < 1e-10
    assert ratios[0] == pytest.approx(math.exp(-0.3), rel=1e-12)
    assert oracle.lambda_init(300) == pytest.approx(lim, abs=1e-15)
    with pytest.raises(ValueError):
        oracle.lambda_init(0)


# ---------------------------------------------------------------------------
# V1
# ---------------------------------------------------------------------------

def v1_rand(seed, T=24, H=1, d=8, dv=16):
    r = rng(seed)
    qk = lambda: r.standard_normal((1, T, H, d))
    return qk(), qk(), qk(), qk(), r.standard_normal((1, T, H, dv))


@pytest.mark.parametrize("causal", [True, False])
def test_v1_lambda_zero_is_softmax_attention(causal):
    q1, k1, q2, k2, v = v1_rand(1, T=37, H=3, d=8, dv=16)
    z = oracle.v1_attention(q1, k1, q2, k2, v, lam=0.0, causal=causal)
    ref = sdpa(q1[0], k1[0], v[0], causal)
    np.testing.assert_allclose(z[0], ref, rtol=0, atol=1e-13)


def test_v1_second_stream_enters_with_minus_lambda():
    # one stream alone is plain attention; the difference is linear in lambda
    q1, k1, q2, k2, v = v1_rand(2, T=19, H=2, d=8, dv=16)
    a1 = sdpa(q1[0], k1[0], v[0], True)
    a2 = sdpa(q2[0], k2[0], v[0], True)
    for lam in (-0.5, 0.2, 0.8, 1.7):
        z = oracle.v1_attention(q1, k1, q2, k2, v, lam)
        np.testing.assert_allclose(z[0], a1 - lam * a2, rtol=0, atol=1e-13)


def test_v1_identical_streams_give_exact_zero():
    q1, k1, _, _, v = v1_rand(3, T=33, H=2, d=16, dv=32)
    z = oracle.v1_attention(q1, k1, q1.copy(), k1.copy(), v, lam=1.0)
    assert np.all(z == 0.0)
    y = oracle.v1_forward(q1, k1, q1.copy(), k1.copy(), v, lam=1.0, lam_init=0.2, eps=1e-12)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("lam", [0.2, 0.7])
def test_v1_uniform_attention_is_prefix_mean(lam):
    # zero keys make every logit 0, so each causal row averages v_0..v_i
    q1, _, q2, _, v = v1_rand(4, T=40, H=2, d=8, dv=16)
    zk = np.zeros_like(q1)
    z = oracle.v1_attention(q1, zk, q2, zk, v, lam)
    n = np.arange(1, 41, dtype=np.float64)[None, :, None, None]
    prefix_mean = np.cumsum(v, axis=1) / n
    np.testing.assert_allclose(z, (1 - lam) * prefix_mean, rtol=0, atol=1e-13)
    lam_init, eps = 0.47, 1e-12
    y = oracle.v1_forward(q1, zk, q2, zk, v, lam, lam_init, eps)
    zz = (1 - lam) * prefix_mean
    expect = (1 - lam_init) * zz / np.sqrt((zz ** 2).mean(-1, keepdims=True) + eps)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-13)


def test_v1_uniform_attention_gain_matches_page_figure():
    # V2 summary §3: uncorrelated RMS-1 values averaged uniformly over n = 8192
    # tokens have context RMS ~ 1/sqrt(n): the norm multiplies by ~90.5.
    fig = GOLDEN["uniform_attention_norm_gain_n8192"]
    n, dv, heads = fig["n"], 64, 256
    r = rng(5)
    ms = []
    zq = np.zeros((n, 4))
    for _ in range(heads):
        v = r.standard_normal((n, dv))
        z = oracle.v1_head(zq, zq, zq, zq, v, lam=0.0, rows=[n - 1])
        ms.append(np.mean(z ** 2))
    gain = 1.0 / math.sqrt(np.mean(ms))
    assert abs(gain - fig["value"]) / fig["value"] < fig["tolerance_rel"]
    assert 1.0 / math.sqrt(n) < math.sqrt(np.mean(ms)) * 1.05  # lower end of [1/sqrt(n), 1)


def test_v1_norm_backward_amplifies_by_page_figure():
    # V2 summary §3: at length 8192 with uniform attention the per-head norm
    # scales its input up ~90.5x, and the gradient through it grows by the same
    # factor: dz = (g - zhat <g, zhat> / dv) / r with zhat = z / r of mean
    # square ~1, so for random g, |dz|^2 ~ |g|^2 (1 - 1/dv) / r^2.  Averaging
    # 1/r^2 rather than r^2 adds the chi-square factor E[dv / chi2_dv] =
    # dv / (dv - 2) to the page's 1/RMS figure.
    fig = GOLDEN["uniform_attention_norm_gain_n8192"]
    n, dv, heads = fig["n"], 64, 256
    r = rng(15)
    zq = np.zeros((n, 4))
    num = den = 0.0
    for _ in range(heads):
        v = r.standard_normal((n, dv))
        z = oracle.v1_head(zq, zq, zq, zq, v, lam=0.0, rows=[n - 1])
        dy = r.standard_normal(z.shape)
        dz, _ = oracle.v1_norm_backward(z, dy, lam_init=0.0, eps=1e-12)
        num += float(np.sum(dz ** 2))
        den += float(np.sum(dy ** 2)) * (1.0 - 1.0 / dv)
    gain = math.sqrt(num / den)
    expect = fig["value"] * math.sqrt(dv / (dv - 2.0))
    assert abs(gain - expect) / expect < fig["tolerance_rel"]


def test_v1_norm_backward_is_orthogonal_to_z_and_scale_invariant():
    # the norm output does not change when z is scaled (eps -> 0), so dz has no
    # component along z and scaling z by c scales dz by 1/c; dw sums s dy z / r
    r = rng(16)
    z = r.standard_normal((5, 7, 32))
    dy = r.standard_normal(z.shape)
    w = 1.0 + 0.1 * r.standard_normal(32)
    dz, dw = oracle.v1_norm_backward(z, dy, 0.3, 0.0, w)
    np.testing.assert_allclose(np.sum(dz * z, axis=-1), 0.0, atol=1e-12)
    dz3, dw3 = oracle.v1_norm_backward(3.0 * z, dy, 0.3, 0.0, w)
    np.testing.assert_allclose(dz3, dz / 3.0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw3, dw, rtol=1e-12, atol=1e-13)
    y = oracle.v1_norm(z, 0.3, 0.0, w)
    np.testing.assert_allclose(dw, np.sum((dy * y / w).reshape(-1, 32), axis=0), rtol=1e-12)


def test_v1_one_hot_maps_select_values():
    # make stream 1 of row i look only at key a, stream 2 only at key b
    T, d, dv, i, a, b = 12, 8, 16, 9, 2, 6
    r = rng(6)
    q1 = np.zeros((1, T, 1, d)); k1 = np.zeros_like(q1)
    q2 = np.zeros_like(q1); k2 = np.zeros_like(q1)
    q1[0, i, 0, 0] = 40.0; k1[0, a, 0, 0] = 40.0
    q2[0, i, 0, 1] = 40.0; k2[0, b, 0, 1] = 40.0
    v = r.standard_normal((1, T, 1, dv))
    lam = 0.35
    z = oracle.v1_attention(q1, k1, q2, k2, v, lam, rows=[i])
    np.testing.assert_allclose(z[0, 0, 0], v[0, a, 0] - lam * v[0, b, 0], rtol=0, atol=1e-12)


def test_v1_first_row_closed_form():
    q1, k1, q2, k2, v = v1_rand(7, T=10, H=3, d=8, dv=16)
    lam, lam_init, eps = 0.6, 0.3555, 1e-6
    w = rng(8).uniform(0.5, 1.5, 16)
    y = oracle.v1_forward(q1, k1, q2, k2, v, lam, lam_init, eps, weight=w, rows=[0])
    z0 = (1 - lam) * v[0, 0]  # one visible key: both maps are exactly 1
    expect = (1 - lam_init) * w * z0 / np.sqrt((z0 ** 2).mean(-1, keepdims=True) + eps)
    np.testing.assert_allclose(y[0, 0], expect, rtol=1e-13, atol=0)


def test_v1_norm_gives_rms_of_scale_per_row_and_head():
    q1, k1, q2, k2, v = v1_rand(9, T=21, H=4, d=8, dv=32)
    lam_init = 0.7008
    y = oracle.v1_forward(q1, k1, q2, k2, v, 0.5, lam_init, eps=0.0)
    rms = np.sqrt((y ** 2).mean(-1))
    np.testing.assert_allclose(rms, 1 - lam_init, rtol=1e-12)


def test_v1_causal_rows_ignore_future_tokens():
    q1, k1, q2, k2, v = v1_rand(10, T=30, H=2, d=8, dv=16)
    y = oracle.v1_forward(q1, k1, q2, k2, v, 0.4, 0.2, 1e-12)
    cut = 17
    k1b, k2b, vb = k1.copy(), k2.copy(), v.copy()
    r = rng(11)
    k1b[:, cut:] = r.standard_normal(k1b[:, cut:].shape)
    k2b[:, cut:] = r.standard_normal(k2b[:, cut:].shape)
    vb[:, cut:] = r.standard_normal(vb[:, cut:].shape)
    yb = oracle.v1_forward(q1, k1b, q2, k2b, vb, 0.4, 0.2, 1e-12)
    assert np.array_equal(y[:, :cut], yb[:, :cut])
    assert not np.allclose(y[:, cut:], yb[:, cut:])


def test_v1_softmax_is_over_keys_shift_invariant():
    # adding one vector to every key shifts each row's logits by a constant
    q1, k1, q2, k2, v = v1_rand(12, T=25, H=1, d=8, dv=16)
    c1, c2 = rng(13).standard_normal(8), rng(14).standard_normal(8)
    z = oracle.v1_attention(q1, k1, q2, k2, v, 0.3)
    zs = oracle.v1_attention(q1, k1 + c1, q2, k2 + c2, v, 0.3)
    np.testing.assert_allclose(z, zs, rtol=0, atol=1e-12)


def brute_v1(q1, k1, q2, k2, v, lam, lam_init, eps):
    """Scalar loops over one (batch, head): the page formula, element by element."""
    T, d = len(q1), len(q1[0])
    dv = len(v[0])
    out = []
    for i in range(T):
        s1 = [sum(q1[i][c] * k1[j][c] for c in range(d)) / math.sqrt(d) for j in range(i + 1)]
        s2 = [sum(q2[i][c] * k2[j][c] for c in range(d)) / math.sqrt(d) for j in range(i + 1)]
        e1 = [math.exp(x - max(s1)) for x in s1]
        e2 = [math.exp(x - max(s2)) for x in s2]
        z = [sum((e1[j] / sum(e1) - lam * e2[j] / sum(e2)) * v[j][c] for j in range(i + 1))
             for c in range(dv)]
        r = math.sqrt(sum(x * x for x in z) / dv + eps)
        out.append([(1 - lam_init) * x / r for x in z])
    return out


@pytest.mark.parametrize("lam", [-0.5, 0.0, 0.2, 1.0, 1.5])
def test_v1_brute_force_tiny(lam):
    r = rng(15)
    T, d, dv = 6, 4, 8
    q1, k1, q2, k2 = (r.standard_normal((1, T, 1, d)) for _ in range(4))
    v = r.standard_normal((1, T, 1, dv))
    y = oracle.v1_forward(q1, k1, q2, k2, v, lam, 0.4, 1e-9)
    ref = brute_v1(q1[0, :, 0].tolist(), k1[0, :, 0].tolist(), q2[0, :, 0].tolist(),
                   k2[0, :, 0].tolist(), v[0, :, 0].tolist(), lam, 0.4, 1e-9)
    np.testing.assert_allclose(y[0, :, 0], np.array(ref), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# V2
# ---------------------------------------------------------------------------

def v2_rand(seed, T=20, Hq=8, Hkv=2, d=8, B=1):
    r = rng(seed)
    return (r.standard_normal((B, T, Hq, d)), r.standard_normal((B, T, Hkv, d)),
            r.standard_normal((B, T, Hkv, d)), r.standard_normal((B, T, Hq // 2)))


@pytest.mark.parametrize("causal", [True, False])
def test_v2_zero_sigmoid_is_gqa_attention_of_even_heads(causal):
    q, k, v, _ = v2_rand(20, T=23, Hq=8, Hkv=2)
    logit = np.full((1, 23, 4), -200.0)  # sigmoid(-200) ~ 1e-87
    out = oracle.v2_forward(q, k, v, logit, causal=causal)
    ref = sdpa(q[0], k[0], v[0], causal, gqa=True)
    np.testing.assert_allclose(out[0], ref[:, 0::2], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 2), (4, 4), (8, 1)])
def test_v2_matches_library_attention_and_logistic(Hq, Hkv):
    q, k, v, logit = v2_rand(21, T=17, Hq=Hq, Hkv=Hkv)
    out = oracle.v2_forward(q, k, v, logit)
    o = sdpa(q[0], k[0], v[0], True, gqa=True)
    ref = o[:, 0::2] - expit(logit[0])[..., None] * o[:, 1::2]
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-13)


def test_v2_identical_pair_with_unit_sigmoid_is_exact_zero():
    # Pairs share their GQA group's K and V (V2 summary §1), so two equal query heads
    # in a pair give equal outputs; sigmoid(40) is exactly 1.0 in float64.
    q, k, v, _ = v2_rand(22, T=26, Hq=16, Hkv=4)
    q[..., 1::2, :] = q[..., 0::2, :]
    logit = np.full((1, 26, 8), 40.0)
    assert oracle.sigmoid(np.array([40.0]))[0] == 1.0
    out = oracle.v2_forward(q, k, v, logit)
    assert np.all(out == 0.0)


def test_v2_one_hot_difference_and_rms_range():
    # V2 summary §4: the difference of two maps spans context RMS in (0, sqrt 2).
    T, d, Hq, Hkv, i, a, b = 10, 8, 2, 1, 8, 1, 5
    r = rng(23)
    q = np.zeros((1, T, Hq, d)); k = np.zeros((1, T, Hkv, d))
    q[0, i, 0, 0] = 40.0; k[0, a, 0, 0] = 40.0
    q[0, i, 1, 1] = 40.0; k[0, b, 0, 1] = 40.0
    v = r.standard_normal((1, T, Hkv, 4096))
    v /= np.sqrt((v ** 2).mean(-1, keepdims=True))  # RMS exactly 1 per token
    for x in (-3.0, 0.0, 2.5):
        logit = np.full((1, T, 1), x)
        out = oracle.v2_forward(q, k, v, logit, rows=[i])[0, 0, 0]
        s = expit(x)
        np.testing.assert_allclose(out, v[0, a, 0] - s * v[0, b, 0], rtol=0, atol=1e-12)
        rms = math.sqrt((out ** 2).mean())
        assert 0.0 < rms < math.sqrt(GOLDEN["context_rms_range_v2"]["upper_sq"])
    # uniform maps in both heads and sigmoid -> 1 drive the output to zero (lower end 0)
    kz = np.zeros_like(k)
    out = oracle.v2_forward(q, kz, v, np.full((1, T, 1), 30.0), rows=[i])
    assert math.sqrt((out ** 2).mean()) < 1e-12


def test_v2_causal_rows_ignore_future_tokens():
    q, k, v, logit = v2_rand(24, T=30)
    out = oracle.v2_forward(q, k, v, logit)
    r = rng(25)
    k2, v2 = k.copy(), v.copy()
    k2[:, 12:] = r.standard_normal(k2[:, 12:].shape)
    v2[:, 12:] = r.standard_normal(v2[:, 12:].shape)
    out2 = oracle.v2_forward(q, k2, v2, logit)
    assert np.array_equal(out[:, :12], out2[:, :12])


def test_v2_varlen_is_per_sequence_attention():
    lens = [5, 1, 9, 0, 14]
    cu = np.cumsum([0] + lens)
    N = cu[-1]
    q, k, v, logit = (a[0] for a in v2_rand(26, T=N, Hq=8, Hkv=2))
    out = oracle.v2_varlen_forward(q, k, v, logit, cu)
    for s in range(len(lens)):
        a, e = cu[s], cu[s + 1]
        if a == e:
            continue
        o = sdpa(q[a:e], k[a:e], v[a:e], True, gqa=True)
        ref = o[:, 0::2] - expit(logit[a:e])[..., None] * o[:, 1::2]
        np.testing.assert_allclose(out[a:e], ref, rtol=0, atol=1e-13)
    # no leakage: rewriting the third sequence leaves the others bit-identical
    k2 = k.copy()
    k2[cu[2]:cu[3]] += 1.0
    out2 = oracle.v2_varlen_forward(q, k2, v, logit, cu)
    keep = np.r_[0:cu[2], cu[3]:N]
    assert np.array_equal(out[keep], out2[keep])
    # a token subset gives the same rows
    sub = np.array([0, 6, 13, 20, N - 1])
    np.testing.assert_array_equal(oracle.v2_varlen_forward(q, k, v, logit, cu, tokens=sub), out[sub])


def test_v2_decode_is_single_query_attention_over_cache():
    B, S, Hq, Hkv, d = 3, 29, 8, 2, 8
    r = rng(27)
    q = r.standard_normal((B, Hq, d))
    kc = r.standard_normal((B, S, Hkv, d)); vc = r.standard_normal((B, S, Hkv, d))
    logit = r.standard_normal((B, Hq // 2))
    lens = np.array([29, 7, 0])
    out = oracle.v2_decode(q, kc, vc, logit, cache_len=lens)
    for b in range(B):
        n = lens[b]
        if n == 0:
            assert np.all(out[b] == 0.0)
            continue
        o = sdpa(q[b][None], kc[b, :n], vc[b, :n], False, gqa=True)[0]
        ref = o[0::2] - expit(logit[b])[:, None] * o[1::2]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-13)
    # decoding the last token equals the last row of causal prefill over the cache
    qs = r.standard_normal((1, S, Hq, d))
    qs[0, -1] = q[0]
    ls = np.zeros((1, S, Hq // 2)); ls[0, -1] = logit[0]
    pre = oracle.v2_forward(qs, kc[:1], vc[:1], ls, rows=[S - 1])
    np.testing.assert_allclose(out[0], pre[0, 0], rtol=0, atol=1e-13)
    # a batch subset with sliced caches
    sub = oracle.v2_decode(q, kc[1:2], vc[1:2], logit, cache_len=lens, batch=[1])
    np.testing.assert_allclose(sub[0], out[1], rtol=0, atol=0)


def brute_v2_row(q, k, v, logit, i, g):
    """Scalar loops for one query row of one sequence."""
    Hq, d = len(q[0]), len(q[0][0])
    dvv = len(v[0][0])
    O = []
    for j in range(Hq):
        kv = j // g
        s = [sum(q[i][j][c] * k[t][kv][c] for c in range(d)) / math.sqrt(d) for t in range(i + 1)]
        e = [math.exp(x - max(s)) for x in s]
        O.append([sum(e[t] / sum(e) * v[t][kv][c] for t in range(i + 1)) for c in range(dvv)])
    res = []
    for p in range(Hq // 2):
        sg = 1.0 / (1.0 + math.exp(-logit[i][p]))
        res.append([O[2 * p][c] - sg * O[2 * p + 1][c] for c in range(dvv)])
    return res


def test_v2_brute_force_tiny():
    q, k, v, logit = v2_rand(28, T=6, Hq=4, Hkv=2, d=4)
    out = oracle.v2_forward(q, k, v, logit)
    for i in range(6):
        ref = brute_v2_row(q[0].tolist(), k[0].tolist(), v[0].tolist(), logit[0].tolist(), i, 2)
        np.testing.assert_allclose(out[0, i], np.array(ref), rtol=1e-11, atol=1e-12)


def test_sigmoid_is_overflow_free_and_symmetric():
    x = np.array([-800.0, -40.0, -1.0, 0.0, 1.0, 40.0, 800.0])
    s = oracle.sigmoid(x)
    assert np.all(np.isfinite(s))
    np.testing.assert_allclose(s, expit(x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(s + oracle.sigmoid(-x), 1.0, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# V2 backward (chain rule through the forward; pinned by finite differences)
# ---------------------------------------------------------------------------

def _v2_loss_and_grads(seed, T, Hq, Hkv, d, causal):
    r = rng(seed)
    q = r.normal(size=(1, T, Hq, d))
    k = r.normal(size=(1, T, Hkv, d))
    v = r.normal(size=(1, T, Hkv, d))
    logit = r.normal(size=(1, T, Hq // 2))
    dout = r.normal(size=(1, T, Hq // 2, d))
    loss = lambda *a: float(np.sum(dout * oracle.v2_forward(*a, causal=causal)))
    return (q, k, v, logit, dout), loss


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (4, 1)])
def test_v2_backward_matches_central_differences_everywhere(causal, Hq, Hkv):
    # Every element of every gradient against a central difference of the forward
    # oracle (step 1e-5: truncation ~1e-10, rounding ~1e-11 at these magnitudes).
    (q, k, v, logit, dout), loss = _v2_loss_and_grads(30 + Hq + Hkv, 5, Hq, Hkv, 3, causal)
    grads = oracle.v2_backward(q, k, v, logit, dout, causal=causal)
    args = [q, k, v, logit]
    h = 1e-5
    for which, g in enumerate(grads):
        fd = np.empty_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-8)


def test_v2_backward_key_gradient_sums_to_zero_over_keys():
    # Adding one vector to every key shifts a query's scores by a constant, which the
    # softmax ignores; so for each KV head the key gradients sum to zero.
    (q, k, v, logit, dout), _ = _v2_loss_and_grads(40, 19, 8, 2, 6, True)
    _, dk, _, _ = oracle.v2_backward(q, k, v, logit, dout)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    assert np.abs(dk).max() > 1e-2


def test_v2_backward_single_token_closed_form():
    # One token: every map is the single weight 1, so S has no influence (dq = dk = 0),
    # out_p = v_kv(p) (1 - sigmoid), and dv sums dout_p (1 - sigmoid(logit_p)) over the
    # pairs of each KV head; dlogit_p = -sigmoid'(logit_p) <dout_p, v_kv>.
    (q, k, v, logit, dout), _ = _v2_loss_and_grads(41, 1, 8, 2, 4, True)
    dq, dk, dv, dlogit = oracle.v2_backward(q, k, v, logit, dout)
    # (zero up to the rounding of dO.v against rowsum(dO o O))
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    s = expit(logit[0, 0])
    for g in range(2):
        pairs = range(2 * g, 2 * g + 2)  # Hq/Hkv = 4 query heads = 2 pairs per KV head
        ref = sum(dout[0, 0, p] * (1 - s[p]) for p in pairs)
        np.testing.assert_allclose(dv[0, 0, g], ref, rtol=1e-14, atol=1e-14)
    for p in range(4):
        ref = -s[p] * (1 - s[p]) * np.dot(dout[0, 0, p], v[0, 0, p // 2])
        np.testing.assert_allclose(dlogit[0, 0, p], ref, rtol=1e-14, atol=1e-15)


def test_v2_backward_zero_upstream_gives_zero():
    (q, k, v, logit, dout), _ = _v2_loss_and_grads(42, 9, 4, 2, 4, True)
    for g in oracle.v2_backward(q, k, v, logit, np.zeros_like(dout)):
        np.testing.assert_array_equal(g, 0.0)


def test_v2_forward_stats_match_library_attention_and_logsumexp():
    # Per-head O against torch SDPA (float64), lse against torch.logsumexp of the
    # masked, scaled scores.
    q, k, v, _ = v2_rand(43, T=21, Hq=8, Hkv=2)
    O, lse = oracle.v2_forward_stats(q, k, v)
    np.testing.assert_allclose(O[0], sdpa(q[0], k[0], v[0], True, gqa=True), rtol=0, atol=1e-13)
    tq = torch.from_numpy(q[0]).permute(1, 0, 2)                       # [Hq, T, d]
    tk = torch.from_numpy(np.repeat(k[0], 4, axis=1)).permute(1, 0, 2)  # GQA groups of 4
    s = tq @ tk.transpose(1, 2) / math.sqrt(q.shape[-1])
    s = s.masked_fill(torch.ones(21, 21, dtype=torch.bool).triu(1), float("-inf"))
    ref = torch.logsumexp(s, dim=-1).T.numpy()
    np.testing.assert_allclose(lse[0], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_v2_backward_query_rows_matches_central_differences(causal):
    # dq and dlogit of selected rows against central differences of the forward oracle
    (q, k, v, logit, dout), loss = _v2_loss_and_grads(44, 6, 8, 2, 3, causal)
    rows = np.array([0, 3, 5])
    dq, dlogit = oracle.v2_backward_query_rows(q[0], k[0], v[0], logit[0], dout[0], rows, causal)
    h = 1e-5
    for which, g in ((0, dq), (3, dlogit)):
        for ridx, r in enumerate(rows):
            for idx in np.ndindex(*g.shape[1:]):
                args = [q, k, v, logit]
                plus = [a.copy() for a in args]
                minus = [a.copy() for a in args]
                plus[which][(0, r) + idx] += h
                minus[which][(0, r) + idx] -= h
                fd = (loss(*plus) - loss(*minus)) / (2 * h)
                assert abs(g[(ridx,) + idx] - fd) <= 2e-8, (which, r, idx)


@pytest.mark.parametrize("causal", [True, False])
def test_v2_backward_key_rows_matches_central_differences(causal):
    # dk and dv of selected keys (all KV heads, and one KV head alone) against
    # central differences of the forward oracle; small row blocks make the
    # row loop run several times
    (q, k, v, logit, dout), loss = _v2_loss_and_grads(45, 7, 8, 2, 3, causal)
    keys = np.array([0, 2, 6])
    h = 1e-5
    for kv_heads in (None, [1]):
        dk, dv = oracle.v2_backward_key_rows(q[0], k[0], v[0], logit[0], dout[0], keys,
                                             kv_heads=kv_heads, causal=causal, row_block=3)
        heads = [0, 1] if kv_heads is None else kv_heads
        for which, g in ((1, dk), (2, dv)):
            for kidx, t in enumerate(keys):
                for slot, kv in enumerate(heads):
                    for c in range(g.shape[-1]):
                        args = [q, k, v, logit]
                        plus = [a.copy() for a in args]
                        minus = [a.copy() for a in args]
                        plus[which][0, t, kv, c] += h
                        minus[which][0, t, kv, c] -= h
                        fd = (loss(*plus) - loss(*minus)) / (2 * h)
                        assert abs(g[kidx, slot, c] - fd) <= 2e-8, (which, t, kv, c)



# ---------------------------------------------------------------------------
# V1 decode
# ---------------------------------------------------------------------------

def test_v1_decode_lambda_zero_is_normalised_single_query_attention():
    # lambda = 0: z is plain attention of the query over the cache (torch SDPA, float64,
    # no mask), then the per-head RMS norm and factor
    r = rng(50)
    B, S, H, d, dv = 2, 37, 3, 8, 16
    q1, q2 = r.normal(size=(B, H, d)), r.normal(size=(B, H, d))
    k1, k2 = r.normal(size=(B, S, H, d)), r.normal(size=(B, S, H, d))
    v = r.normal(size=(B, S, H, dv))
    out = oracle.v1_decode(q1, q2, k1, k2, v, 0.0, 0.3, 0.0)
    for b in range(B):
        z = sdpa(q1[b][None], k1[b], v[b], False)[0]                     # [H, dv]
        ref = 0.7 * z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True))
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_v1_decode_brute_force_tiny():
    # scalar loops with math.exp: both maps, the difference, the norm and the weight
    r = rng(51)
    B, S, H, d, dv = 2, 5, 2, 3, 4
    q1, q2 = r.normal(size=(B, H, d)), r.normal(size=(B, H, d))
    k1, k2 = r.normal(size=(B, S, H, d)), r.normal(size=(B, S, H, d))
    v = r.normal(size=(B, S, H, dv))
    w = r.normal(size=dv)
    lens = np.array([5, 3])
    lam, li, eps = 0.6, 0.2, 1e-3
    out = oracle.v1_decode(q1, q2, k1, k2, v, lam, li, eps, weight=w, cache_len=lens)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            def smax(q, k):
                s = [sum(q[t] * k[j, t] for t in range(d)) / math.sqrt(d) for j in range(n)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                return [x / sum(e) for x in e]
            p1, p2 = smax(q1[b, h], k1[b, :, h]), smax(q2[b, h], k2[b, :, h])
            z = [sum((p1[j] - lam * p2[j]) * v[b, j, h, c] for j in range(n)) for c in range(dv)]
            rr = math.sqrt(sum(x * x for x in z) / dv + eps)
            for c in range(dv):
                assert abs(out[b, h, c] - (1 - li) * w[c] * z[c] / rr) < 1e-12


def test_v1_decode_empty_cache_gives_zeros():
    r = rng(52)
    q = r.normal(size=(1, 2, 4))
    k = r.normal(size=(1, 6, 2, 4))
    v = r.normal(size=(1, 6, 2, 8))
    out = oracle.v1_decode(q, q, k, k, v, 0.2, 0.2, 1e-12, cache_len=np.array([0]))
    np.testing.assert_array_equal(out, 0.0)



# ---------------------------------------------------------------------------
# V1 backward (chain rule through the forward and the norm; finite differences)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_v1_backward_matches_central_differences_everywhere(causal):
    r = rng(60)
    B, T, H, d, dv = 1, 5, 2, 3, 6
    q1, k1, q2, k2 = (r.normal(size=(B, T, H, d)) for _ in range(4))
    v = r.normal(size=(B, T, H, dv))
    dy = r.normal(size=(B, T, H, dv))
    w = r.normal(size=dv)
    lam, li, eps = 0.45, 0.2, 1e-3
    grads = oracle.v1_backward(q1, k1, q2, k2, v, lam, li, eps, dy, weight=w, causal=causal)

    def loss(q1_, k1_, q2_, k2_, v_, lam_, w_):
        return float(np.sum(dy * oracle.v1_forward(q1_, k1_, q2_, k2_, v_, lam_, li, eps, weight=w_,
                                                   causal=causal)))
    args = [q1, k1, q2, k2, v, lam, w]
    h = 1e-5
    for which in (0, 1, 2, 3, 4, 6):
        g = grads[which if which < 5 else 6]
        fd = np.empty_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() if isinstance(a, np.ndarray) else a for a in args]
            minus = [a.copy() if isinstance(a, np.ndarray) else a for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=5e-8)
    lp = args.copy(); lp[5] = lam + h
    lm = args.copy(); lm[5] = lam - h
    assert abs(grads[5] - (loss(*lp) - loss(*lm)) / (2 * h)) < 5e-8


def test_v1_backward_key_gradients_sum_to_zero_and_norm_is_scale_free():
    # each map's key gradients sum to zero over keys (softmax shift invariance); the norm
    # makes y invariant to scaling V (eps = 0), so <dv, v> = 0 over each (b, h)
    r = rng(61)
    B, T, H, d, dv = 1, 17, 2, 4, 8
    q1, k1, q2, k2 = (r.normal(size=(B, T, H, d)) for _ in range(4))
    v = r.normal(size=(B, T, H, dv))
    dy = r.normal(size=(B, T, H, dv))
    dq1, dk1, dq2, dk2, dvv, dlam, dw = oracle.v1_backward(q1, k1, q2, k2, v, 0.3, 0.2, 0.0, dy)
    np.testing.assert_allclose(dk1.sum(axis=1), 0.0, atol=1e-11)
    np.testing.assert_allclose(dk2.sum(axis=1), 0.0, atol=1e-11)
    for h in range(H):
        assert abs(np.sum(dvv[0, :, h] * v[0, :, h])) < 1e-9 * np.sum(np.abs(dvv[0, :, h] * v[0, :, h]))


def test_v1_backward_zero_upstream_gives_zero():
    r = rng(62)
    q = r.normal(size=(1, 6, 1, 4))
    v = r.normal(size=(1, 6, 1, 8))
    g = oracle.v1_backward(q, q, q, q, v, 0.2, 0.2, 1e-6, np.zeros_like(v))
    for x in g:
        np.testing.assert_array_equal(x, 0.0)


# ---------------------------------------------------------------------------
# Projections either side of the V2 attention
# ---------------------------------------------------------------------------

def test_projections_match_brute_force_loops():
    r = rng(21)
    x = r.standard_normal((5, 12))
    w = r.standard_normal((3, 12))
    got = oracle.v2_lambda_logits(x, w)
    for n in range(5):
        for p in range(3):
            assert abs(got[n, p] - math.fsum(x[n, c] * w[p, c] for c in range(12))) < 1e-12
    a = r.standard_normal((4, 16))
    wo = r.standard_normal((6, 16))
    y = oracle.out_projection(a, wo)
    for n in range(4):
        for j in range(6):
            assert abs(y[n, j] - math.fsum(a[n, c] * wo[j, c] for c in range(16))) < 1e-12


def test_difference_before_projection_equals_negated_pair_weights():
    # V2 summary §7: a 2h-head model could express the difference by giving the
    # two heads of a pair exactly opposite output weights.  With sigma = 1 the
    # V2 output projected by W equals the 2h-head outputs projected by
    # [W_p, -W_p] per pair (sigma < 1 scales the odd head's block instead).
    r = rng(22)
    T, Hq, Hkv, d, dm = 9, 8, 2, 4, 5
    q = r.standard_normal((1, T, Hq, d))
    k = r.standard_normal((1, T, Hkv, d))
    v = r.standard_normal((1, T, Hkv, d))
    h = Hq // 2
    for logit_val, sig in ((60.0, 1.0), (0.3, float(expit(0.3)))):
        logit = np.full((1, T, h), logit_val)
        out = oracle.v2_forward(q, k, v, logit).reshape(T, h * d)
        heads = oracle.v2_heads(q[0], k[0], v[0]).reshape(T, Hq * d)
        w = r.standard_normal((dm, h * d))
        w_base = np.zeros((dm, Hq * d))
        for p in range(h):
            w_base[:, (2 * p) * d:(2 * p + 1) * d] = w[:, p * d:(p + 1) * d]
            w_base[:, (2 * p + 1) * d:(2 * p + 2) * d] = -sig * w[:, p * d:(p + 1) * d]
        np.testing.assert_allclose(oracle.out_projection(out, w),
                                   oracle.out_projection(heads, w_base), rtol=1e-12, atol=1e-12)


def test_output_projection_saving_matches_page_figures():
    # count weights by building the projections as torch modules (independent of
    # the oracle's arithmetic), then compare with the page's half and ~25 %
    fig = GOLDEN["v2_output_projection_saving"]
    for d_model, h, hkv, d in ((4096, 32, 8, 128), (4096, 32, 4, 128), (8192, 64, 8, 128)):
        c = oracle.v2_attention_param_counts(d_model, h, hkv, d)
        mods = {"q": torch.nn.Linear(d_model, 2 * h * d, bias=False, device="meta"),
                "k": torch.nn.Linear(d_model, hkv * d, bias=False, device="meta"),
                "v": torch.nn.Linear(d_model, hkv * d, bias=False, device="meta"),
                "lam": torch.nn.Linear(d_model, h, bias=False, device="meta"),
                "o_v2": torch.nn.Linear(h * d, d_model, bias=False, device="meta"),
                "o_base": torch.nn.Linear(2 * h * d, d_model, bias=False, device="meta")}
        n = {k: m.weight.numel() for k, m in mods.items()}
        assert c["v2"] == n["q"] + n["k"] + n["v"] + n["lam"] + n["o_v2"]
        assert c["base"] == n["q"] + n["k"] + n["v"] + n["o_base"]
        assert c["o_v2"] / c["o_base"] == fig["o_projection_fraction_kept"]
        base = n["q"] + n["k"] + n["v"] + n["o_base"]
        assert c["o_saving_frac_of_base"] == (n["o_base"] - n["o_v2"]) / base
        # The page's ~25 % holds when the query and output projections hold the
        # module's weights; the K and V projections (2 hkv d of the 4 h d + 2 hkv d
        # base columns) move the exact saving h / (4h + 2hkv) below 1/4 by
        # (2hkv/h) / (4 (4 + 2hkv/h)) <= hkv / (8h).
        assert abs(c["o_saving_frac_of_base"] - fig["attention_params_saved_frac"]) <= fig["tolerance_abs"] + hkv / (8 * h)
    small_kv = oracle.v2_attention_param_counts(4096, 32, 1, 128)
    assert abs(small_kv["o_saving_frac_of_base"] - fig["attention_params_saved_frac"]) < fig["tolerance_abs"]


# ---------------------------------------------------------------------------
# Grouped Differential Attention (the reading in the oracle: blocks of r
# signal heads and one noise head inside a GQA group)
# ---------------------------------------------------------------------------

def _gda_brute_row(q, k, v, logit, i, g, r, scale):
    """Scalar loops with math.exp for query row i of one sequence."""
    Hq = len(q[0])
    d = len(q[0][0])
    O = []
    for j in range(Hq):
        kv = j // g
        s = [sum(q[i][j][c] * k[t][kv][c] for c in range(d)) * scale for t in range(i + 1)]
        e = [math.exp(x - max(s)) for x in s]
        O.append([sum(e[t] / sum(e) * v[t][kv][c] for t in range(i + 1)) for c in range(d)])
    res = []
    for s_ in range(Hq // (r + 1) * r):
        blk, pos = divmod(s_, r)
        sg = 1.0 / (1.0 + math.exp(-logit[i][s_]))
        res.append([O[blk * (r + 1) + pos][c] - sg * O[blk * (r + 1) + r][c] for c in range(d)])
    return res


@pytest.mark.parametrize("ratio,Hq,Hkv", [(3, 8, 2), (4, 10, 2), (3, 8, 1)])
def test_gda_brute_force_tiny(ratio, Hq, Hkv):
    r = rng(60 + ratio + Hq)
    T, d = 5, 3
    q, k, v = r.normal(size=(1, T, Hq, d)), r.normal(size=(1, T, Hkv, d)), r.normal(size=(1, T, Hkv, d))
    nout = Hq // (ratio + 1) * ratio
    logit = r.normal(size=(1, T, nout))
    out = oracle.gda_forward(q, k, v, logit, ratio)
    assert out.shape == (1, T, nout, d)
    for i in range(T):
        ref = _gda_brute_row(q[0].tolist(), k[0].tolist(), v[0].tolist(), logit[0].tolist(), i,
                             Hq // Hkv, ratio, 1.0 / math.sqrt(d))
        np.testing.assert_allclose(out[0, i], np.array(ref), rtol=1e-11, atol=1e-12)


def test_gda_one_to_one_is_v2():
    q, k, v, logit = v2_rand(61, T=17, Hq=8, Hkv=2)
    np.testing.assert_array_equal(oracle.gda_forward(q, k, v, logit, 1), oracle.v2_forward(q, k, v, logit))


def test_gda_sigmoid_zero_is_gqa_attention_of_the_signal_heads():
    # logit -800: sigmoid is 0 to double precision, so every output head is the
    # plain GQA attention of its signal head (torch SDPA, float64, enable_gqa)
    r = rng(62)
    T, Hq, Hkv, d, ratio = 19, 8, 2, 8, 3
    q, k, v = r.normal(size=(1, T, Hq, d)), r.normal(size=(1, T, Hkv, d)), r.normal(size=(1, T, Hkv, d))
    logit = np.full((1, T, 6), -800.0)
    out = oracle.gda_forward(q, k, v, logit, ratio)
    ref = sdpa(q[0], k[0], v[0], True, gqa=True)          # [T, Hq, d]
    sig, _ = oracle.gda_heads(Hq, ratio)
    assert sig == [0, 1, 2, 4, 5, 6]
    np.testing.assert_allclose(out[0], ref[:, sig], rtol=0, atol=1e-13)


def test_gda_identical_signal_and_noise_heads_give_zero():
    # every head of a block carries the same query and sigmoid(40) = 1 - 4e-18:
    # the subtraction cancels (to rounding of the sigmoid)
    r = rng(63)
    T, Hkv, d, ratio = 12, 2, 4, 4
    q1 = r.normal(size=(1, T, Hkv * 2, 1, d))
    q = np.repeat(q1, ratio + 1, axis=3).reshape(1, T, Hkv * 2 * (ratio + 1), d)
    k, v = r.normal(size=(1, T, Hkv, d)), r.normal(size=(1, T, Hkv, d))
    logit = np.full((1, T, Hkv * 2 * ratio), 40.0)
    out = oracle.gda_forward(q, k, v, logit, ratio)
    assert np.abs(out).max() <= 1e-15 * np.abs(v).max() * 10


def test_gda_decode_is_the_last_prefill_row():
    r = rng(64)
    T, Hq, Hkv, d, ratio = 23, 8, 2, 8, 3
    q, k, v = r.normal(size=(1, T, Hq, d)), r.normal(size=(1, T, Hkv, d)), r.normal(size=(1, T, Hkv, d))
    logit = r.normal(size=(1, T, 6))
    pre = oracle.gda_forward(q, k, v, logit, ratio)
    dec = oracle.gda_decode(q[:, -1], k, v, logit[:, -1], ratio)
    np.testing.assert_allclose(dec[0], pre[0, -1], rtol=0, atol=1e-13)
    # an empty cache gives zeros
    assert np.all(oracle.gda_decode(q[:, -1], k, v, logit[:, -1], ratio, cache_len=np.array([0])) == 0)


def test_gda_rejects_blocks_across_gqa_groups():
    q, k, v, logit = v2_rand(65, T=4, Hq=8, Hkv=4)   # groups of 2 heads: a 4-head block cannot fit
    with pytest.raises(ValueError):
        oracle.gda_forward(q, k, v, np.zeros((1, 4, 6)), 3)
