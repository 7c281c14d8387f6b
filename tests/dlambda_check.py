"""Bounds for the V1 backward's dlambda, shared by the GPU parity tests and the
CPU check that the bounds reject wrong answers.

dlambda = -sum_i <dz_i, O2_i> runs over every row and head, and its terms
cancel heavily: <dz_i, z_i> = 0 by the norm's scale invariance, and O1 ~ O2
when both maps are near-uniform, so sum|terms| is 10^3 to 10^4 times |dlambda|
at the workloads' input scale.  Two bounds follow (no figure on the pages; the
derivation is from the arithmetic):

* Backward on the oracle's forward state (O1, O2, lse given in fp32): the
  kernel rounds each term once in fp32 and sums in a fixed tree, so
  |err| <= 2e-3 |ref| + 2^-24 sum|terms|  (one fp32 ulp of the magnitude
  of the whole sum; measured errors are ~1e-5 |ref|, well inside).

* End to end (the kernel's own training forward feeds the backward): the
  forward's O carries fp16-rounded P (2^-11 relative per weight), and the
  change of O moves dlambda to first order by <G, dO>, G = d(dlambda)/dO
  from the oracle.  With the measured forward error dO = O_kernel - O_oracle
  and the elementwise errors taken as independent, that change has standard
  deviation sqrt(sum (G dO)^2); the bound is 6 of those plus the oracle-state
  bound.  When it is not below |ref| / 2 the end-to-end value cannot tell
  dlambda from zero, and the oracle-state check alone is decisive: the test
  says so in its output.
"""
from __future__ import annotations

import math

import numpy as np
import torch

U32 = 2.0 ** -24          # fp32 unit roundoff
REL_ORACLE_STATE = 2e-3   # relative part of the oracle-state bound
SIGMAS = 6.0              # width of the end-to-end bound in standard deviations


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def dlambda_terms(O1, O2, dy, lam, li, eps, weight=None) -> np.ndarray:
    """Terms -dz_ic O2_ic of dlambda (fp64, from the oracle's O), [..., dv]."""
    O1, O2, dy = _f64(O1), _f64(O2), _f64(dy)
    w = 1.0 if weight is None else _f64(weight)
    z = O1 - lam * O2
    r = np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    g = (1.0 - li) * w * dy
    dz = g / r - z * np.sum(g * z, axis=-1, keepdims=True) / (z.shape[-1] * r ** 3)
    return -dz * O2


def dlambda_sensitivity(O1, O2, dy, lam, li, eps, weight=None):
    """G1, G2 = d(dlambda)/dO1, d(dlambda)/dO2 at the oracle's O (float64 autograd of
    the same chain rule dlambda_terms writes out)."""
    o1 = torch.from_numpy(_f64(O1)).requires_grad_(True)
    o2 = torch.from_numpy(_f64(O2)).requires_grad_(True)
    dyt = torch.from_numpy(_f64(dy))
    w = 1.0 if weight is None else torch.from_numpy(_f64(weight))
    z = o1 - lam * o2
    r = torch.sqrt((z * z).mean(-1, keepdim=True) + eps)
    g = (1.0 - li) * w * dyt
    dz = g / r - z * (g * z).sum(-1, keepdim=True) / (z.shape[-1] * r ** 3)
    (-(dz * o2).sum()).backward()
    return o1.grad.numpy(), o2.grad.numpy()


def oracle_state_bound(ref, terms) -> float:
    return REL_ORACLE_STATE * abs(float(ref)) + U32 * float(np.sum(np.abs(terms)))


def end_to_end_bound(ref, terms, G1, G2, dO1, dO2) -> tuple[float, float]:
    """(bound, sigma): sigma = sqrt(sum (G dO)^2) from the measured forward error."""
    sigma = math.sqrt(float(np.sum((G1 * _f64(dO1)) ** 2) + np.sum((G2 * _f64(dO2)) ** 2)))
    return SIGMAS * sigma + oracle_state_bound(ref, terms), sigma


def decisive(bound, ref) -> bool:
    """A bound tells dlambda from 0 and from -ref only below |ref| / 2."""
    return bound < 0.5 * abs(float(ref))
