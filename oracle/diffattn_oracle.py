"""fp64 CPU oracle for differential attention (V1 and V2) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The library (HIP kernels, C ABI and its Python binding)
never imports, links or calls it, and this module imports nothing from the
library: the two share no code.  Inputs come in as arrays (numpy or anything
``numpy.asarray`` accepts) and are promoted exactly to float64.

What is computed, and where it is stated
-----------------------------------------
* V1 differential attention -- "Differential Transformer | ICLR 2025 Oral" blog
  (dainus.ai), section "Differential Attention: 빼기의 힘": the output is
  (softmax(Q1 K1^T / sqrt d) - lambda * softmax(Q2 K2^T / sqrt d)) V, with the
  two maps from independent query/key halves.  The value head is twice as wide
  as the query/key head ("파라미터 효율성" on the same page; V2 summary §1).
* lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)) -- same blog, section "λ의 역할과 학습".
* V1 post-processing -- "Differential Transformer V2" summary (pogovet.com),
  상세 정리 §1: after the subtraction each head is RMS-normalised and then
  multiplied by a factor set by the layer's initial lambda; that factor is
  (1 - lambda_init).
* V2 -- same summary, §1 and §4: one attention call over 2h query heads whose
  key/value heads are shared within GQA groups; the outputs are split into
  even/odd heads and the odd one, scaled by sigmoid of a per-token, per-head
  coefficient, is subtracted from the even one, leaving h*d columns.  No norm
  and no scale follow.
* V2 decode -- same summary, §2: the KV heads and cache are those of a
  standard GQA model; a decode step is the V2 formula for one new query row
  against every cached position.  V1 decode is the V1 formula (with its norm)
  for one new query row against the cached K1, K2 and V.

Readings where the pages are silent (each one is an argument, not a constant)
----------------------------------------------------------------------------
* sqrt(d) uses the query/key head dim d, not the value width.
* Causal masking keeps keys j <= i (diagonal included); a packed (varlen)
  batch never attends across sequence boundaries.
* The RMS norm runs over the value channels of one (token, head):
  y = (1 - lambda_init) * w * z / sqrt(mean(z^2) + eps); w defaults to ones.
* Pairs are (2p, 2p+1); query head j reads KV head j // (Hq / Hkv).
* sigmoid(x) = 1 / (1 + e^-x), evaluated in its overflow-free form.
* A decode sequence with no cached positions gives a zero output.

V2 backward (training)
----------------------
The pages quote V2's throughput for pretraining but print no gradient.  The
backward functions below are the chain rule through the V2 forward above,
written term by term: with sigma = sigmoid(logit), the even head of pair p
receives dO_2p = dOut_p and the odd head dO_2p+1 = -sigma * dOut_p;
dlogit_p = -sigma (1 - sigma) <dOut_p, O_2p+1>; each head then takes the usual
softmax-attention backward (dP = dO V^T, dS = P o (dP - rowsum(dO o O)),
dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO), and the gradients of the
query heads sharing a KV head add up.  Pinned against central finite
differences of ``v2_forward``.

V1 backward (training): the chain rule through the V1 forward and its norm
(``v1_head_backward``), likewise pinned by finite differences.

Parity status: every public function here is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

_ROW_BLOCK = 256


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: go through float32 (exact for bf16/fp32)
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def lambda_init(layer: int) -> float:
    """Initial lambda of (1-based) layer ``layer``: 0.8 - 0.6 * exp(-0.3 * (layer - 1)).

    Blog "Differential Transformer | ICLR 2025 Oral", section "λ의 역할과 학습".
    """
    if int(layer) != layer or layer < 1:
        raise ValueError("layer is 1-based")
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def sigmoid(x) -> np.ndarray:
    """Logistic function 1 / (1 + e^-x) without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, with the row maximum subtracted first.

    Entries equal to -inf (masked keys) get weight exactly 0.
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _attention_map(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, scale: float,
                   causal: bool) -> np.ndarray:
    """softmax(q k^T * scale) for the query positions ``rows`` against keys 0..n-1."""
    s = (q_rows @ k.T) * scale
    if causal:
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    return softmax_rows(s)


# ---------------------------------------------------------------------------
# V1
# ---------------------------------------------------------------------------

def v1_head(q1, k1, q2, k2, v, lam: float, rows=None, causal: bool = True) -> np.ndarray:
    """Differential attention z for one (batch, head) slice.

    q1, k1, q2, k2: [T, d]; v: [T, dv].  Returns z[rows] = (P1 - lam * P2) v, [R, dv],
    where P1, P2 are the two softmax maps (blog, "Differential Attention: 빼기의 힘").
    The difference map is formed first, literally as written on the page.
    """
    q1, k1, q2, k2, v = (_f64(a) for a in (q1, k1, q2, k2, v))
    T, d = q1.shape
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(d)
    out = np.empty((rows.size, v.shape[1]))
    for r0 in range(0, rows.size, _ROW_BLOCK):
        rr = rows[r0:r0 + _ROW_BLOCK]
        p1 = _attention_map(q1[rr], k1, rr, scale, causal)
        p2 = _attention_map(q2[rr], k2, rr, scale, causal)
        diff_map = p1 - lam * p2
        out[r0:r0 + rr.size] = diff_map @ v
    return out


def v1_norm(z, lam_init: float, eps: float, weight=None) -> np.ndarray:
    """Per-head RMS norm over the value channels, then the (1 - lambda_init) factor.

    V2 summary §1 (the V1 recap): normalise each head, then multiply by a factor
    set by the layer's initial lambda.  z: [..., dv]; weight: [dv] or None (ones).
    """
    z = _f64(z)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    y = z / np.sqrt(ms + eps)
    if weight is not None:
        y = y * _f64(weight)
    return (1.0 - lam_init) * y


def v1_norm_backward(z, dy, lam_init: float, eps: float, weight=None):
    """Backward of ``v1_norm``: gradients of sum(dy * y) with respect to z and the weight.

    The chain rule through y = s w z / r (V2 summary §1, the V1 recap), with
    s = 1 - lam_init, r = sqrt(mean(z^2) + eps) over the dv channels and g = s w dy:
        dz = g / r - z <g, z> / (dv r^3),   dw = sum over rows of s dy z / r.
    z, dy: [..., dv].  Returns (dz [..., dv], dw [dv]).
    """
    z, dy = _f64(z), _f64(dy)
    dvw = z.shape[-1]
    w = np.ones(dvw) if weight is None else _f64(weight)
    r = np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    s = 1.0 - lam_init
    g = s * w * dy
    dz = g / r - z * np.sum(g * z, axis=-1, keepdims=True) / (dvw * r ** 3)
    dw = np.sum((s * dy * z / r).reshape(-1, dvw), axis=0)
    return dz, dw


def v1_attention(q1, k1, q2, k2, v, lam: float, causal: bool = True, rows=None) -> np.ndarray:
    """z for every (batch, head): inputs [B, T, H, d] / [B, T, H, dv] -> [B, R, H, dv]."""
    q1, k1, q2, k2, v = (_f64(a) for a in (q1, k1, q2, k2, v))
    B, T, H, _ = q1.shape
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, rows.size, H, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            out[b, :, h] = v1_head(q1[b, :, h], k1[b, :, h], q2[b, :, h], k2[b, :, h],
                                   v[b, :, h], lam, rows, causal)
    return out


def v1_forward(q1, k1, q2, k2, v, lam: float, lam_init: float, eps: float, weight=None,
               causal: bool = True, rows=None) -> np.ndarray:
    """Full V1 attention output y = (1 - lam_init) * w * z / rms(z): [B, R, H, dv]."""
    z = v1_attention(q1, k1, q2, k2, v, lam, causal, rows)
    return v1_norm(z, lam_init, eps, weight)


def v1_head_backward(q1, k1, q2, k2, v, lam: float, lam_init: float, eps: float, dy, weight=None,
                     causal: bool = True):
    """Gradients of sum(dy * y) for one (batch, head) slice of the V1 forward.

    The chain rule through ``v1_head`` and ``v1_norm`` (the pages print no gradient):
    with y = s w z / r, s = 1 - lam_init, r = sqrt(mean(z^2) + eps), g = s w dy,
        dz = g / r - z <g, z> / (dv r^3),      dw += s dy z / r,
        dO1 = dz,  dO2 = -lam dz,  dlam = -sum <dz, O2>,
    and for each map k the softmax-attention backward
        dP = dO_k v^T,  dS = P_k o (dP - rowsum(dO_k o O_k)),
        dq_k = dS k_k / sqrt(d),  dk_k = dS^T q_k / sqrt(d),  dv += P_k^T dO_k.
    q1, k1, q2, k2 [T, d]; v, dy [T, dv].
    Returns (dq1, dk1, dq2, dk2, dv, dlam, dw).
    """
    q1, k1, q2, k2, v, dy = (_f64(a) for a in (q1, k1, q2, k2, v, dy))
    T, d = q1.shape
    rows = np.arange(T)
    scale = 1.0 / math.sqrt(d)
    p1 = _attention_map(q1, k1, rows, scale, causal)
    p2 = _attention_map(q2, k2, rows, scale, causal)
    o1, o2 = p1 @ v, p2 @ v
    z = o1 - lam * o2
    dz, dw = v1_norm_backward(z, dy, lam_init, eps, weight)
    dlam = -float(np.sum(dz * o2))
    grads = []
    dv = np.zeros_like(v)
    for p, o, q, k, do in ((p1, o1, q1, k1, dz), (p2, o2, q2, k2, -lam * dz)):
        dp = do @ v.T
        ds = p * (dp - np.sum(do * o, axis=-1, keepdims=True))
        grads.append((scale * (ds @ k), scale * (ds.T @ q)))
        dv += p.T @ do
    (dq1, dk1), (dq2, dk2) = grads
    return dq1, dk1, dq2, dk2, dv, dlam, dw


def v1_backward(q1, k1, q2, k2, v, lam: float, lam_init: float, eps: float, dy, weight=None,
                causal: bool = True):
    """Batch version of ``v1_head_backward``: inputs [B, T, H, d] / [B, T, H, dv], dy like v.

    Returns (dq1, dk1, dq2, dk2, dv, dlam, dw); dlam and dw sum over every (b, t, h).
    """
    q1, k1, q2, k2, v, dy = (_f64(a) for a in (q1, k1, q2, k2, v, dy))
    B, T, H, _ = q1.shape
    out = [np.zeros_like(q1), np.zeros_like(k1), np.zeros_like(q2), np.zeros_like(k2),
           np.zeros_like(v)]
    dlam, dw = 0.0, np.zeros(v.shape[-1])
    for b in range(B):
        for h in range(H):
            g = v1_head_backward(q1[b, :, h], k1[b, :, h], q2[b, :, h], k2[b, :, h], v[b, :, h],
                                 lam, lam_init, eps, dy[b, :, h], weight, causal)
            for i in range(5):
                out[i][b, :, h] = g[i]
            dlam += g[5]
            dw += g[6]
    return (*out, dlam, dw)


def v1_decode(q1, q2, k1_cache, k2_cache, v_cache, lam: float, lam_init: float, eps: float,
              weight=None, cache_len=None, batch=None) -> np.ndarray:
    """One V1 decode step: q1, q2 [B, H, d]; caches k1/k2 [B, S, H, d], v [B, S, H, dv].

    Entry b's query attends (non-causally) to cache positions 0 .. cache_len[b]-1 (all
    S when ``cache_len`` is None) with both maps, then the V1 norm and factor: the V1
    formula for a single query row (blog section "Differential Attention: 빼기의 힘";
    V2 summary §1 for the norm).  An entry with no cached positions gives zeros.
    ``batch`` selects entries; the caches may then hold only those entries.
    Returns [B', H, dv].
    """
    q1, q2 = _f64(q1), _f64(q2)
    B, H, d = q1.shape
    batch = list(range(B)) if batch is None else [int(b) for b in batch]
    S = k1_cache.shape[1]
    out = np.zeros((len(batch), H, v_cache.shape[-1]))
    sliced = k1_cache.shape[0] == len(batch) and len(batch) != B
    for i, b in enumerate(batch):
        n = S if cache_len is None else int(np.asarray(cache_len)[b])
        if n <= 0:
            continue
        cb = i if sliced else b
        k1b, k2b, vb = _f64(k1_cache[cb, :n]), _f64(k2_cache[cb, :n]), _f64(v_cache[cb, :n])
        for h in range(H):
            z = v1_head(q1[b, h][None], k1b[:, h], q2[b, h][None], k2b[:, h], vb[:, h], lam,
                        rows=np.array([0]), causal=False)
            out[i, h] = v1_norm(z, lam_init, eps, weight)[0]
    return out


# ---------------------------------------------------------------------------
# V2
# ---------------------------------------------------------------------------

def gqa_kv_head(j: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head j: contiguous groups of Hq / Hkv query heads."""
    return j // (Hq // Hkv)


def v2_heads(q, k, v, rows=None, causal: bool = True, scale: float | None = None) -> np.ndarray:
    """Plain softmax attention of every query head over its GQA KV head, one sequence.

    q: [T, Hq, d]; k, v: [T, Hkv, d].  Returns O: [R, Hq, d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.empty((rows.size, Hq, v.shape[-1]))
    for j in range(Hq):
        kv = gqa_kv_head(j, Hq, Hkv)
        for r0 in range(0, rows.size, _ROW_BLOCK):
            rr = rows[r0:r0 + _ROW_BLOCK]
            p = _attention_map(q[rr, j], k[:, kv], rr, scale, causal)
            out[r0:r0 + rr.size, j] = p @ v[:, kv]
    return out


def v2_combine(O, logit) -> np.ndarray:
    """out[:, p] = O[:, 2p] - sigmoid(logit[:, p]) * O[:, 2p+1]  (V2 summary §1, §4).

    O: [R, 2h, d]; logit: [R, h].  Returns [R, h, d].
    """
    O, logit = _f64(O), _f64(logit)
    if O.shape[1] % 2:
        raise ValueError("an even number of query heads is required")
    sig = sigmoid(logit)
    return O[:, 0::2] - sig[..., None] * O[:, 1::2]


def v2_sequence(q, k, v, logit, rows=None, causal: bool = True,
                scale: float | None = None) -> np.ndarray:
    """V2 output for one sequence: q [T, 2h, d], k/v [T, Hkv, d], logit [T, h] -> [R, h, d]."""
    logit = _f64(logit)
    T = logit.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    O = v2_heads(q, k, v, rows, causal, scale)
    return v2_combine(O, logit[rows])


def v2_forward(q, k, v, logit, causal: bool = True, scale: float | None = None,
               rows=None) -> np.ndarray:
    """Padded batch: q [B, T, 2h, d], k/v [B, T, Hkv, d], logit [B, T, h] -> [B, R, h, d]."""
    q, k, v, logit = _f64(q), _f64(k), _f64(v), _f64(logit)
    B, T = q.shape[:2]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, rows.size, q.shape[2] // 2, v.shape[-1]))
    for b in range(B):
        out[b] = v2_sequence(q[b], k[b], v[b], logit[b], rows, causal, scale)
    return out


def v2_varlen_forward(q, k, v, logit, cu_seqlens, causal: bool = True,
                      scale: float | None = None, tokens=None) -> np.ndarray:
    """Packed batch: q [N, 2h, d], k/v [N, Hkv, d], logit [N, h], cu_seqlens [nseq+1].

    Each sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends only
    within itself.  ``tokens`` (global indices) selects output rows; default all.
    Returns [len(tokens), h, d].
    """
    q, k, v, logit = _f64(q), _f64(k), _f64(v), _f64(logit)
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    N = q.shape[0]
    tokens = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((tokens.size, q.shape[1] // 2, v.shape[-1]))
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        sel = np.nonzero((tokens >= a) & (tokens < e))[0]
        if sel.size == 0:
            continue
        out[sel] = v2_sequence(q[a:e], k[a:e], v[a:e], logit[a:e], tokens[sel] - a, causal, scale)
    return out


def v2_decode(q, k_cache, v_cache, logit, cache_len=None, scale: float | None = None,
              batch=None) -> np.ndarray:
    """One decode step: q [B, 2h, d], caches [B, S, Hkv, d], logit [B, h] -> [B', h, d].

    Entry b attends (non-causally) to cache positions 0 .. cache_len[b]-1 (all S when
    ``cache_len`` is None); an entry with no cached positions gives zeros.  ``batch``
    selects entries (default all); the caches may then hold only those entries
    (``k_cache.shape[0] == len(batch)``) to bound host memory.
    """
    q, logit = _f64(q), _f64(logit)
    B = q.shape[0]
    batch = list(range(B)) if batch is None else [int(b) for b in batch]
    h = q.shape[1] // 2
    S = k_cache.shape[1]
    out = np.zeros((len(batch), h, v_cache.shape[-1]))
    sliced = k_cache.shape[0] == len(batch) and len(batch) != B
    for i, b in enumerate(batch):
        n = S if cache_len is None else int(np.asarray(cache_len)[b])
        if n <= 0:
            continue
        cb = i if sliced else b
        kb, vb = _f64(k_cache[cb, :n]), _f64(v_cache[cb, :n])
        O = v2_heads(q[b][None], kb, vb, rows=np.array([0]), causal=False, scale=scale)
        out[i] = v2_combine(O, logit[b][None])[0]
    return out


# ---------------------------------------------------------------------------
# V2 backward (the chain rule through v2_forward; see the module docstring)
# ---------------------------------------------------------------------------

def v2_sequence_backward(q, k, v, logit, dout, causal: bool = True, scale: float | None = None):
    """Gradients of sum(dout * v2_sequence(q, k, v, logit)) for one sequence.

    q [T, 2h, d], k/v [T, Hkv, d], logit [T, h], dout [T, h, d].
    Returns (dq [T, 2h, d], dk [T, Hkv, d], dv [T, Hkv, d], dlogit [T, h]).
    """
    q, k, v, logit, dout = (_f64(a) for a in (q, k, v, logit, dout))
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv or Hq % 2:
        raise ValueError("Hq must be even and a multiple of Hkv")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(T)
    sig = sigmoid(logit)                                   # [T, h]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlogit = np.zeros_like(logit)
    for j in range(Hq):
        kv = gqa_kv_head(j, Hq, Hkv)
        p = _attention_map(q[:, j], k[:, kv], rows, scale, causal)   # P_j  [T, T]
        o = p @ v[:, kv]                                             # O_j  [T, d]
        if j % 2 == 0:
            do = dout[:, j // 2]                                     # dO of the even head
        else:
            do = -sig[:, j // 2, None] * dout[:, j // 2]             # dO of the odd head
            dlogit[:, j // 2] = -sig[:, j // 2] * (1.0 - sig[:, j // 2]) * np.sum(
                dout[:, j // 2] * o, axis=-1)
        dp = do @ v[:, kv].T                                         # dL/dP
        dsum = np.sum(do * o, axis=-1, keepdims=True)                # rowsum(dO o O)
        ds = p * (dp - dsum)                                         # dL/dS (softmax backward)
        dq[:, j] = scale * (ds @ k[:, kv])
        dk[:, kv] += scale * (ds.T @ q[:, j])
        dv[:, kv] += p.T @ do
    return dq, dk, dv, dlogit


def v2_backward(q, k, v, logit, dout, causal: bool = True, scale: float | None = None):
    """Padded batch: q [B, T, 2h, d], k/v [B, T, Hkv, d], logit [B, T, h], dout [B, T, h, d].

    Returns (dq, dk, dv, dlogit) shaped like (q, k, v, logit).
    """
    q, k, v, logit, dout = (_f64(a) for a in (q, k, v, logit, dout))
    outs = [v2_sequence_backward(q[b], k[b], v[b], logit[b], dout[b], causal, scale)
            for b in range(q.shape[0])]
    return tuple(np.stack([o[i] for o in outs]) for i in range(4))


def v2_forward_stats(q, k, v, causal: bool = True, scale: float | None = None):
    """Per-head outputs and log-sum-exp of one padded batch, as a training forward keeps them.

    Returns (O [B, T, 2h, d], lse [B, T, 2h]) with lse = log sum_k exp(q.k * scale) over
    the visible keys (natural log).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.empty((B, T, Hq, v.shape[-1]))
    lse = np.empty((B, T, Hq))
    rows = np.arange(T)
    for b in range(B):
        for j in range(Hq):
            kv = gqa_kv_head(j, Hq, Hkv)
            s = (q[b, :, j] @ k[b, :, kv].T) * scale
            if causal:
                s = np.where(rows[None, :] > rows[:, None], -np.inf, s)
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=-1, keepdims=True)
            O[b, :, j] = (e / l) @ v[b, :, kv]
            lse[b, :, j] = (m + np.log(l))[:, 0]
    return O, lse


def v2_backward_query_rows(q, k, v, logit, dout, rows, causal: bool = True,
                           scale: float | None = None):
    """dq and dlogit of one sequence at the query positions ``rows`` only.

    Same chain rule as ``v2_sequence_backward``, restricted to the rows: a row's
    dq and dlogit need only its own attention row, so this runs at any length.
    q [T, 2h, d], k/v [T, Hkv, d], logit [T, h], dout [T, h, d] ->
    (dq [R, 2h, d], dlogit [R, h]).
    """
    q, k, v, logit, dout = (_f64(a) for a in (q, k, v, logit, dout))
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    sig = sigmoid(logit[rows])                               # [R, h]
    dq = np.empty((rows.size, Hq, d))
    dlogit = np.empty((rows.size, Hq // 2))
    for j in range(Hq):
        kv = gqa_kv_head(j, Hq, Hkv)
        p = _attention_map(q[rows, j], k[:, kv], rows, scale, causal)   # [R, T]
        o = p @ v[:, kv]
        if j % 2 == 0:
            do = dout[rows, j // 2]
        else:
            do = -sig[:, j // 2, None] * dout[rows, j // 2]
            dlogit[:, j // 2] = -sig[:, j // 2] * (1.0 - sig[:, j // 2]) * np.sum(
                dout[rows, j // 2] * o, axis=-1)
        dp = do @ v[:, kv].T
        ds = p * (dp - np.sum(do * o, axis=-1, keepdims=True))
        dq[:, j] = scale * (ds @ k[:, kv])
    return dq, dlogit


def v2_backward_key_rows(q, k, v, logit, dout, keys, kv_heads=None, causal: bool = True,
                         scale: float | None = None, row_block: int = 1024):
    """dk and dv of one sequence at the key positions ``keys`` only.

    Same chain rule as ``v2_sequence_backward``, restricted to the columns
    ``keys`` of every attention map: dk[t] = scale * sum_i dS[i, t] q_i and
    dv[t] = sum_i P[i, t] dO_i, summed over the query heads of the KV head.
    Each query row still needs its whole softmax row (for P's normaliser) and
    its output O_i (for rowsum(dO o O)), so the cost is that of the forward
    over the rows that can see the keys (i >= min(keys) when causal); rows are
    taken ``row_block`` at a time to bound memory.  ``kv_heads`` (default all)
    selects the KV heads to compute.
    q [T, 2h, d], k/v [T, Hkv, d], logit [T, h], dout [T, h, d] ->
    (dk [K, len(kv_heads), d], dv [K, len(kv_heads), d]).
    """
    q, k, v, logit, dout = (_f64(a) for a in (q, k, v, logit, dout))
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv or Hq % 2:
        raise ValueError("Hq must be even and a multiple of Hkv")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    keys = np.asarray(keys, dtype=np.int64)
    kv_heads = list(range(Hkv)) if kv_heads is None else [int(x) for x in kv_heads]
    sig = sigmoid(logit)                                     # [T, h]
    dk = np.zeros((keys.size, len(kv_heads), d))
    dv = np.zeros((keys.size, len(kv_heads), v.shape[-1]))
    first = int(keys.min()) if causal and keys.size else 0
    for slot, kv in enumerate(kv_heads):
        for j in (j for j in range(Hq) if gqa_kv_head(j, Hq, Hkv) == kv):
            for r0 in range(first, T, row_block):
                rows = np.arange(r0, min(r0 + row_block, T))
                p = _attention_map(q[rows, j], k[:, kv], rows, scale, causal)   # [R, T]
                o = p @ v[:, kv]                                             # O_j of the rows
                if j % 2 == 0:
                    do = dout[rows, j // 2]
                else:
                    do = -sig[rows, j // 2, None] * dout[rows, j // 2]
                pk = p[:, keys]                                              # P at the keys
                dpk = do @ v[keys, kv].T                                     # dP at the keys
                dsk = pk * (dpk - np.sum(do * o, axis=-1, keepdims=True))    # dS at the keys
                dk[:, slot] += scale * (dsk.T @ q[rows, j])
                dv[:, slot] += pk.T @ do
    return dk, dv


# ---------------------------------------------------------------------------
# Grouped Differential Attention (unequal signal : noise head counts)
# ---------------------------------------------------------------------------
#
# The blog "Differential Transformer | ICLR 2025 Oral" (section "같은 문제,
# 다른 접근") names Grouped Differential Attention as the follow-up that splits
# the heads unevenly, r signal heads per noise head (3:1 or 4:1), and gives no
# formula.  Reading (the V2 form of the subtraction, which the V2 summary §1
# gives for r = 1): the query heads form blocks of r + 1 consecutive heads, r
# signal heads then one noise head, every block inside one GQA group (so its
# heads share K and V, as V2 requires of a pair); each signal head subtracts
# its block's noise head, scaled by the sigmoid of its own per-token
# coefficient.  r = 1 is V2.

def gda_heads(Hq: int, ratio: int):
    """(signal head, noise head) query-head indices of each output head s."""
    if ratio < 1 or Hq % (ratio + 1):
        raise ValueError("Hq must be a multiple of ratio + 1")
    nout = Hq // (ratio + 1) * ratio
    sig = [(s // ratio) * (ratio + 1) + s % ratio for s in range(nout)]
    noise = [(s // ratio) * (ratio + 1) + ratio for s in range(nout)]
    return sig, noise


def gda_combine(O, logit, ratio: int) -> np.ndarray:
    """out[:, s] = O[:, sig(s)] - sigmoid(logit[:, s]) * O[:, noise(s)].

    O: [R, Hq, d]; logit: [R, Hq r / (r + 1)].  Returns [R, Hq r / (r + 1), d].
    """
    O, logit = _f64(O), _f64(logit)
    sig, noise = gda_heads(O.shape[1], ratio)
    return O[:, sig] - sigmoid(logit)[..., None] * O[:, noise]


def gda_sequence(q, k, v, logit, ratio: int, rows=None, causal: bool = True,
                 scale: float | None = None) -> np.ndarray:
    """One sequence: q [T, Hq, d], k/v [T, Hkv, d], logit [T, Hq r / (r + 1)]."""
    q = _f64(q)
    Hq, Hkv = q.shape[1], _f64(k).shape[1]
    if (Hq // Hkv) % (ratio + 1):
        raise ValueError("each block of ratio + 1 heads must lie in one GQA group")
    logit = _f64(logit)
    rows = np.arange(logit.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = v2_heads(q, k, v, rows, causal, scale)
    return gda_combine(O, logit[rows], ratio)


def gda_forward(q, k, v, logit, ratio: int, causal: bool = True, scale: float | None = None,
                rows=None) -> np.ndarray:
    """Padded batch: q [B, T, Hq, d], k/v [B, T, Hkv, d], logit [B, T, nout] -> [B, R, nout, d]."""
    q, k, v, logit = _f64(q), _f64(k), _f64(v), _f64(logit)
    B, T = q.shape[:2]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    return np.stack([gda_sequence(q[b], k[b], v[b], logit[b], ratio, rows, causal, scale)
                     for b in range(B)])


def gda_decode(q, k_cache, v_cache, logit, ratio: int, cache_len=None,
               scale: float | None = None) -> np.ndarray:
    """One decode step: q [B, Hq, d], caches [B, S, Hkv, d], logit [B, nout] -> [B, nout, d].

    Entry b attends to cache positions 0 .. cache_len[b]-1 (all S when None);
    an entry with no cached positions gives zeros.
    """
    q, logit = _f64(q), _f64(logit)
    B, Hq = q.shape[:2]
    S = k_cache.shape[1]
    nout = Hq // (ratio + 1) * ratio
    out = np.zeros((B, nout, v_cache.shape[-1]))
    for b in range(B):
        n = S if cache_len is None else int(np.asarray(cache_len)[b])
        if n <= 0:
            continue
        O = v2_heads(q[b][None], _f64(k_cache[b, :n]), _f64(v_cache[b, :n]), rows=np.array([0]),
                     causal=False, scale=scale)
        out[b] = gda_combine(O, logit[b][None], ratio)[0]
    return out


# ---------------------------------------------------------------------------
# The projections on either side of the V2 attention
# ---------------------------------------------------------------------------

def v2_lambda_logits(x, w_lambda) -> np.ndarray:
    """Per-token, per-pair coefficients projected from the layer input.

    V2 summary §1: the coefficient that scales the second head of a pair comes
    from a projection of X, one per token and pair, and passes through a
    sigmoid where it is used.  This returns the projection (the logits):
    x [N, d_model], w_lambda [h, d_model] (one weight row per pair) -> [N, h].
    """
    return _f64(x) @ _f64(w_lambda).T


def out_projection(attn_out, w_o) -> np.ndarray:
    """Output projection of the attention output: attn_out [N, K] @ w_o^T.

    V2 summary §1 and §7: after the subtraction each token carries h*d
    columns, so the output projection has the baseline's shape (h*d in,
    d_model out).  w_o [d_model, K] (one row per output feature) -> [N, d_model].
    """
    return _f64(attn_out) @ _f64(w_o).T


def v2_attention_param_counts(d_model: int, h: int, hkv: int, d: int) -> dict:
    """Weight counts of one attention module, V2 against a 2h-head GQA baseline.

    V2 summary §1, §7: V2 has 2h query heads of dim d (as the baseline with the
    same 2h*d query width), hkv shared key/value heads, a per-pair coefficient
    projection (d_model -> h), and an output projection from h*d columns (the
    difference is taken before it); the baseline projects all 2h*d columns.
    Returns the counts per projection and the saving as a fraction of the
    baseline module.
    """
    q = d_model * 2 * h * d
    kv = 2 * d_model * hkv * d
    lam = d_model * h
    o_v2 = h * d * d_model
    o_base = 2 * h * d * d_model
    v2 = q + kv + lam + o_v2
    base = q + kv + o_base
    return {"q": q, "kv": kv, "lambda": lam, "o_v2": o_v2, "o_base": o_base, "v2": v2,
            "base": base, "o_saving": o_base - o_v2,
            "o_saving_frac_of_base": (o_base - o_v2) / base}
