"""Seeded synthetic inputs for the differential-attention workloads.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds no attention arithmetic: only random draws, the
sequence-length draw for packed batches, and rounding to the storage dtype.

By default every tensor is drawn on the CPU with ``torch.Generator`` so that
the same seed gives the same values on any machine.  Large tensors are drawn
one leading index (batch entry or token block) at a time, each from its own
derived seed, so that a slice can be regenerated without materialising the
whole tensor on the host.  With ``device=`` a GPU, the same recipe runs on that
device's generator instead (same seeds, different but equally deterministic
values); callers that check such inputs read them back from the device.

Workload shapes follow the models the method's pages discuss: a 12-head,
d_model 3072 V1 model whose value heads are twice as wide as its query/key
heads, and V2 GQA models with 64 query heads (32 even/odd pairs) over 8 KV
heads at sequence length 8192.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

INV_SQRT_128 = 1.0 / math.sqrt(128.0)


def slice_seed(seed: int, index: int) -> int:
    """Seed of slice ``index`` of a tensor drawn with base seed ``seed``."""
    return (int(seed) * 1_000_003 + int(index)) % (2**63 - 1)


def normal_slice(shape, seed: int, index: int, std: float = 1.0, mean: float = 0.0,
                 dtype: torch.dtype = torch.bfloat16, device=None) -> torch.Tensor:
    """One slice: fp32 N(0,1) draw, times ``std`` plus ``mean`` in fp32, rounded to ``dtype``."""
    dev = torch.device("cpu") if device is None else torch.device(device)
    g = torch.Generator(device=dev).manual_seed(slice_seed(seed, index))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=dev)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x if dtype == torch.float32 else x.to(dtype)


def normal(shape, seed: int, std: float = 1.0, mean: float = 0.0,
           dtype: torch.dtype = torch.bfloat16, device=None) -> torch.Tensor:
    """A tensor drawn slice by slice along its first axis (see :func:`normal_slice`)."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        out[i] = normal_slice(shape[1:], seed, i, std, mean, dtype, device)
    return out


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Sequence lengths for a packed batch.

    Lengths are drawn uniformly from [lo, hi] with ``numpy.random.default_rng(seed)``
    and appended (the last one cut short) until they sum to ``total``; so the
    last sequence may be shorter than ``lo``.
    """
    rng = np.random.default_rng(seed)
    lens: list[int] = []
    acc = 0
    while acc < total:
        x = int(rng.integers(lo, hi + 1))
        x = min(x, total - acc)
        lens.append(x)
        acc += x
    return lens


def cu_seqlens_of(lengths) -> list[int]:
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class V1Workload:
    """V1 differential attention prefill: Q1,K1,Q2,K2 [B,T,H,d], V [B,T,H,dv]."""
    name: str
    B: int
    T: int
    H: int
    d: int
    dv: int
    dtype: torch.dtype
    std: float
    layers: tuple
    seeds: tuple  # q1, k1, q2, k2, v
    eps: float = 1e-12
    causal: bool = True

    def with_shape(self, **kw) -> "V1Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return V1Workload(**d)


@dataclass(frozen=True)
class V2Workload:
    """V2 GQA prefill, padded [B,T,*] or packed varlen [total,*] when ``lengths`` is set."""
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    std: float
    seeds: tuple  # q, k, v, logit
    logit_mean: float = 0.0
    logit_std: float = 1.0
    lengths: tuple | None = None
    causal: bool = True
    ratio: int = 1  # signal heads per noise head (grouped variant; 1 = pairs)

    @property
    def n_out(self) -> int:
        """Output heads (and logits per token): blocks of ratio + 1 query heads give ratio each."""
        return self.Hq // (self.ratio + 1) * self.ratio

    def with_shape(self, **kw) -> "V2Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return V2Workload(**d)


@dataclass(frozen=True)
class DecodeWorkload:
    """V2 decode step: q [B,Hq,d], caches [B,S,Hkv,d], logits [B,Hq/2]."""
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    d: int
    std: float
    seeds: tuple  # q, k_cache, v_cache, logit
    cache_lens: tuple | None = None
    ratio: int = 1  # signal heads per noise head (grouped variant; 1 = pairs)

    @property
    def n_out(self) -> int:
        return self.Hq // (self.ratio + 1) * self.ratio

    def with_shape(self, **kw) -> "DecodeWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return DecodeWorkload(**d)


V1_FP32_SMALL = V1Workload(
    name="v1_fp32_causal_b1_h1_t128_d64_dv128", B=1, T=128, H=1, d=64, dv=128,
    dtype=torch.float32, std=1.0, layers=(1,), seeds=(101, 102, 103, 104, 105))

V1_BF16 = V1Workload(
    name="v1_bf16_causal_b4_h12_t4096_d128_dv256", B=4, T=4096, H=12, d=128, dv=256,
    dtype=torch.bfloat16, std=INV_SQRT_128, layers=tuple(range(1, 29)),
    seeds=(201, 202, 203, 204, 205))

V2_PREFILL = V2Workload(
    name="v2_prefill_bf16_causal_b2_t8192_hq64_hkv8_d128", B=2, T=8192, Hq=64, Hkv=8, d=128,
    std=INV_SQRT_128, seeds=(301, 302, 303, 304))

V2_DECODE = DecodeWorkload(
    name="v2_decode_bf16_b64_s32768_hq64_hkv8_d128", B=64, S=32768, Hq=64, Hkv=8, d=128,
    std=INV_SQRT_128, seeds=(401, 402, 403, 404))

@dataclass(frozen=True)
class V1DecodeWorkload:
    """V1 decode step: q1, q2 [B,H,d], caches k1, k2 [B,S,H,d] and v [B,S,H,dv]."""
    name: str
    B: int
    S: int
    H: int
    d: int
    dv: int
    std: float
    seeds: tuple  # q1, q2, k1_cache, k2_cache, v_cache
    layer: int = 1
    eps: float = 1e-12
    cache_lens: tuple | None = None

    def with_shape(self, **kw) -> "V1DecodeWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return V1DecodeWorkload(**d)


# The V1 model of the headline prefill (12 heads, d 128, dv 256) decoding against a
# 32768-entry cache, batch 32: 12.9 GB of K1, K2 and V.
V1_DECODE = V1DecodeWorkload(
    name="v1_decode_bf16_b32_s32768_h12_d128_dv256", B=32, S=32768, H=12, d=128, dv=256,
    std=INV_SQRT_128, seeds=(601, 602, 603, 604, 605))

VARLEN_SEED = 501
VARLEN_TOTAL = 65536
VARLEN_LO, VARLEN_HI = 512, 16384

V2_VARLEN = V2Workload(
    name="v2_varlen_bf16_causal_total65536_hq64_hkv8_d128", B=1, T=VARLEN_TOTAL, Hq=64, Hkv=8,
    d=128, std=INV_SQRT_128, seeds=(502, 503, 504, 505), logit_mean=2.0, logit_std=1.0,
    lengths=tuple(varlen_lengths(VARLEN_TOTAL, VARLEN_LO, VARLEN_HI, VARLEN_SEED)))

# One sequence decoding against the full 32768-entry cache (a small-batch decode step).
V2_DECODE_B1 = V2_DECODE.with_shape(name="v2_decode_bf16_b1_s32768_hq64_hkv8_d128", B=1)

# A packed batch of many short sequences: 2048 x 32 tokens (65536 in all).
V2_VARLEN_SHORT = V2_VARLEN.with_shape(name="v2_varlen_bf16_causal_2048x32_hq64_hkv8_d128",
                                       lengths=(32,) * 2048)

# Grouped variant at the V2 prefill's and decode's shapes: in each GQA group of 8
# query heads, two blocks of 3 signal heads and 1 noise head (48 output heads);
# and 4:1 with 80 query heads over the same 8 KV heads (two blocks of 5 per group,
# 64 output heads).
GDA_PREFILL_R3 = V2_PREFILL.with_shape(name="gda_prefill_bf16_causal_b2_t8192_hq64_hkv8_d128_r3",
                                       ratio=3)
GDA_PREFILL_R4 = V2_PREFILL.with_shape(name="gda_prefill_bf16_causal_b2_t8192_hq80_hkv8_d128_r4",
                                       Hq=80, ratio=4)
GDA_DECODE_R3 = V2_DECODE.with_shape(name="gda_decode_bf16_b64_s32768_hq64_hkv8_d128_r3", ratio=3)

WORKLOADS = {w.name: w for w in (V1_FP32_SMALL, V1_BF16, V2_PREFILL, V2_DECODE, V2_VARLEN,
                                  V1_DECODE, V2_DECODE_B1, V2_VARLEN_SHORT, GDA_PREFILL_R3,
                                  GDA_PREFILL_R4, GDA_DECODE_R3)}


# ---------------------------------------------------------------------------
# Generators (CPU tensors; callers move them to a device)
# ---------------------------------------------------------------------------

def v1_inputs(w: V1Workload, device=None) -> dict:
    sq, sk, sq2, sk2, sv = w.seeds
    qk_shape = (w.B, w.T, w.H, w.d)
    return dict(
        q1=normal(qk_shape, sq, w.std, dtype=w.dtype, device=device),
        k1=normal(qk_shape, sk, w.std, dtype=w.dtype, device=device),
        q2=normal(qk_shape, sq2, w.std, dtype=w.dtype, device=device),
        k2=normal(qk_shape, sk2, w.std, dtype=w.dtype, device=device),
        v=normal((w.B, w.T, w.H, w.dv), sv, w.std, dtype=w.dtype, device=device),
    )


V1_DY_SEED = 206  # upstream gradient of the V1 backward workload (B4 T4096 H12 d128 dv256)


def v1_dy(w: V1Workload, seed: int = V1_DY_SEED, device=None) -> torch.Tensor:
    """Upstream gradient dL/dy [B,T,H,dv] fp32, iid N(0,1)."""
    return normal((w.B, w.T, w.H, w.dv), seed, 1.0, dtype=torch.float32, device=device)


def v2_inputs(w: V2Workload, device=None) -> dict:
    """Padded: q [B,T,Hq,d] ...; packed (``w.lengths`` set): q [total,Hq,d], plus cu_seqlens."""
    sq, sk, sv, sl = w.seeds
    h = w.n_out
    if w.lengths is None:
        lead = (w.B, w.T)
        return dict(
            q=normal(lead + (w.Hq, w.d), sq, w.std, device=device),
            k=normal(lead + (w.Hkv, w.d), sk, w.std, device=device),
            v=normal(lead + (w.Hkv, w.d), sv, w.std, device=device),
            logit=normal(lead + (h,), sl, w.logit_std, w.logit_mean, dtype=torch.float32,
                         device=device),
            cu_seqlens=None,
        )
    total = int(sum(w.lengths))
    # packed tensors are drawn in blocks of 1024 tokens (one derived seed per block)
    def packed(width, seed, std, mean=0.0, dtype=torch.bfloat16):
        blk = 1024
        nb = (total + blk - 1) // blk
        t = normal((nb, blk) + width, seed, std, mean, dtype, device)
        return t.reshape((nb * blk,) + width)[:total].contiguous()
    return dict(
        q=packed((w.Hq, w.d), sq, w.std),
        k=packed((w.Hkv, w.d), sk, w.std),
        v=packed((w.Hkv, w.d), sv, w.std),
        logit=packed((h,), sl, w.logit_std, w.logit_mean, dtype=torch.float32),
        cu_seqlens=torch.tensor(cu_seqlens_of(w.lengths), dtype=torch.int32, device=device),
    )


@dataclass(frozen=True)
class ProjWorkload:
    """The projections either side of the V2 attention: N tokens, model width
    d_model (= h * d, the baseline's attention width), h pairs, h * d columns
    after the subtraction."""
    name: str
    N: int
    d_model: int
    h: int
    d: int
    seeds: tuple  # x, w_lambda, attn_out, w_o


# the V2 prefill workload's tokens (B2 x T8192), 32 pairs of d = 128
V2_PROJ = ProjWorkload(name="v2_proj_bf16_n16384_dmodel4096_h32_d128", N=16384, d_model=4096,
                       h=32, d=128, seeds=(701, 702, 703, 704))


def _rows(n_rows: int, n_cols: int, seed: int, std: float, device=None) -> torch.Tensor:
    """[n_rows, n_cols] bf16 drawn in blocks of 256 rows (one derived seed per block)."""
    nb = (n_rows + 255) // 256
    t = normal((nb, 256, n_cols), seed, std, device=device)
    return t.reshape(nb * 256, n_cols)[:n_rows].contiguous()


def proj_inputs(w: ProjWorkload, device=None) -> dict:
    """x [N, d_model] N(0,1); w_lambda [h, d_model] and w_o [d_model, h*d] N(0, 1/fan_in);
    attn_out [N, h*d] N(0,1); all bf16."""
    sx, sl, sa, so = w.seeds
    hd = w.h * w.d
    return dict(
        x=_rows(w.N, w.d_model, sx, 1.0, device),
        w_lambda=_rows(w.h, w.d_model, sl, 1.0 / math.sqrt(w.d_model), device),
        attn_out=_rows(w.N, hd, sa, 1.0, device),
        w_o=_rows(w.d_model, hd, so, 1.0 / math.sqrt(hd), device),
    )


DOUT_SEED = 305  # upstream gradient of the V2 backward workload (B2 T8192 Hq64 Hkv8 d128)


def v2_varlen_dout(w: V2Workload, seed: int = DOUT_SEED, device=None) -> torch.Tensor:
    """Upstream gradient [N,Hq/2,d] bf16 of a packed batch, iid N(0,1), drawn in
    blocks of 1024 tokens like the packed inputs."""
    total = int(sum(w.lengths))
    nb = (total + 1023) // 1024
    t = normal((nb, 1024, w.Hq // 2, w.d), seed, 1.0, device=device)
    return t.reshape(nb * 1024, w.Hq // 2, w.d)[:total].contiguous()


def v2_dout(w: V2Workload, seed: int = DOUT_SEED, device=None) -> torch.Tensor:
    """Upstream gradient dL/dout [B,T,Hq/2,d] bf16, iid N(0,1) (padded batches)."""
    return normal((w.B, w.T, w.Hq // 2, w.d), seed, 1.0, device=device)


def decode_small_inputs(w: DecodeWorkload, device=None) -> dict:
    """Decode inputs for the query, logits and lengths (the caches come from :func:`decode_cache_slice`)."""
    sq, sk, sv, sl = w.seeds
    h = w.n_out
    lens = None if w.cache_lens is None else torch.tensor(w.cache_lens, dtype=torch.int32,
                                                          device=device)
    return dict(
        q=normal((w.B, w.Hq, w.d), sq, w.std, device=device),
        logit=normal((w.B, h), sl, 1.0, dtype=torch.float32, device=device),
        cache_len=lens,
    )


def decode_cache_slice(w: DecodeWorkload, b: int, which: str, device=None) -> torch.Tensor:
    """Cache slice [S, Hkv, d] of batch entry ``b``; ``which`` is 'k' or 'v'."""
    seed = w.seeds[1] if which == "k" else w.seeds[2]
    return normal_slice((w.S, w.Hkv, w.d), seed, b, w.std, device=device)


def decode_inputs(w: DecodeWorkload, device=None) -> dict:
    """All decode inputs, drawn on ``device`` (CPU when None), caches one batch entry at a time."""
    out = decode_small_inputs(w, device)
    dev = torch.device("cpu") if device is None else torch.device(device)
    kc = torch.empty((w.B, w.S, w.Hkv, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    for b in range(w.B):
        kc[b].copy_(decode_cache_slice(w, b, "k", device))
        vc[b].copy_(decode_cache_slice(w, b, "v", device))
    out["k_cache"], out["v_cache"] = kc, vc
    return out


def v1_decode_inputs(w: V1DecodeWorkload, device=None) -> dict:
    """All V1 decode inputs on ``device`` (CPU when None); caches drawn one batch entry at a time."""
    sq1, sq2, sk1, sk2, sv = w.seeds
    dev = torch.device("cpu") if device is None else torch.device(device)
    out = dict(
        q1=normal((w.B, w.H, w.d), sq1, w.std, device=device),
        q2=normal((w.B, w.H, w.d), sq2, w.std, device=device),
        cache_len=None if w.cache_lens is None else torch.tensor(w.cache_lens, dtype=torch.int32,
                                                                 device=device),
    )
    for name, seed, width in (("k1_cache", sk1, w.d), ("k2_cache", sk2, w.d), ("v_cache", sv, w.dv)):
        t = torch.empty((w.B, w.S, w.H, width), dtype=torch.bfloat16, device=dev)
        for b in range(w.B):
            t[b].copy_(normal_slice((w.S, w.H, width), seed, b, w.std, device=device))
        out[name] = t
    return out
