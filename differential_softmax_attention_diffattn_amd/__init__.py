"""Differential attention (DIFF V1 / V2) on AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/diffattn.h``: every function
here only checks and marshals torch tensors (device, dtype, shape,
contiguity), allocates outputs/workspaces with torch when the caller does not
pass them, and calls the HIP library on torch's current stream.  All of the
arithmetic runs in the library's kernels; there is no fallback path.

    v1_fwd      V1: (softmax(Q1K1^T/sqrt d) - lambda softmax(Q2K2^T/sqrt d)) V,
                per-head RMS norm, (1 - lambda_init) factor
    v2_fwd      V2: GQA attention over 2h query heads, O_even - sigmoid(logit) O_odd
                (padded or packed/varlen batches)
    v2_decode   V2 decode step against a KV cache
    v2_decode_noalloc
                the same without a workspace (partials in a library-owned array)
    v1_decode   V1 decode step against cached K1, K2 and V (with the norm)
    v2_fwd_train / v2_bwd
                V2 training forward (also keeps per-head O and log-sum-exp) and
                the backward: gradients of q, k, v and the lambda logits
    v2_varlen_fwd_train / v2_varlen_bwd
                the same for packed (varlen) batches
    v1_fwd_train / v1_bwd
                V1 training forward (also keeps per-map O and log-sum-exp) and
                the backward through the norm: gradients of q1, k1, q2, k2, v,
                lambda and the norm weight
    v2_lambda_proj / out_proj
                the projections either side of the V2 attention: coefficient
                logits from the layer input, and the output projection of the
                h*d columns left after the subtraction
    lambda_init 0.8 - 0.6 exp(-0.3 (l - 1))
"""
from __future__ import annotations

from . import _lib
from ._lib import DIFFATTN_BF16, DIFFATTN_F32, DiffAttnError  # noqa: F401

__all__ = [
    "v1_fwd",
    "v2_fwd",
    "v2_decode",
    "v2_decode_noalloc",
    "gda_fwd",
    "gda_decode",
    "v1_decode",
    "v2_fwd_train",
    "v2_bwd",
    "v1_fwd_train",
    "v1_bwd",
    "v2_varlen_fwd_train",
    "v2_varlen_bwd",
    "v2_lambda_proj",
    "out_proj",
    "lambda_init",
    "v1_workspace_bytes",
    "v2_decode_workspace_bytes",
    "gda_decode_workspace_bytes",
    "v1_decode_workspace_bytes",
    "v2_bwd_workspace_bytes",
    "v1_bwd_workspace_bytes",
    "DiffAttnError",
]


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DIFFATTN_F32
    if t.dtype == torch.bfloat16:
        return DIFFATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_tensor(name, t, dtype=None, dim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _outputs(fn, outs, specs, dev):
    """Output tensors of ``fn``: the caller's ``outs`` (checked against ``specs``,
    a list of (name, shape, dtype)) or new ones."""
    torch = _torch()
    if outs is None:
        return [torch.empty(shape, dtype=dt, device=dev) for _, shape, dt in specs]
    outs = list(outs)
    if len(outs) != len(specs):
        raise ValueError(f"{fn}: outs must hold {len(specs)} tensors ({', '.join(n for n, _, _ in specs)})")
    for t, (name, shape, dt) in zip(outs, specs):
        _check_tensor(name, t, dtype=dt, dim=len(shape), device=dev)
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn}: {name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return outs


def lambda_init(layer: int) -> float:
    """Initial lambda of 1-based layer ``layer`` (computed by the library, fp32)."""
    v = _lib.load().diffattn_lambda_init(int(layer))
    if v != v:  # NaN
        _lib.check("diffattn_lambda_init", -1)
    return v


def v1_workspace_bytes(B, T, H, d, dv, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(_lib.load().diffattn_v1_workspace_bytes(B, T, H, d, dv, code))


def v1_fwd(q1, k1, q2, k2, v, lam: float, lambda_init: float, eps: float = 1e-12, weight=None,
           causal: bool = True, out=None, workspace=None):
    """DIFF V1 forward.  q1,k1,q2,k2: [B,T,H,d]; v: [B,T,H,dv] (fp32 or bf16) -> out [B,T,H,dv] fp32."""
    torch = _torch()
    dev = q1.device
    _check_tensor("q1", q1, dim=4)
    for n, t in (("k1", k1), ("q2", q2), ("k2", k2)):
        _check_tensor(n, t, dtype=q1.dtype, dim=4, device=dev)
        if t.shape != q1.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != q1 shape {tuple(q1.shape)}")
    _check_tensor("v", v, dtype=q1.dtype, dim=4, device=dev)
    B, T, H, d = q1.shape
    if tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"v shape {tuple(v.shape)} does not match q1 {tuple(q1.shape)}")
    dv = v.shape[3]
    if weight is not None:
        _check_tensor("weight", weight, dtype=torch.float32, dim=1, device=dev)
        if weight.shape[0] != dv:
            raise ValueError("weight must have dv entries")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _check_tensor("out", out, dtype=torch.float32, dim=4, device=dev)
    if tuple(out.shape) != (B, T, H, dv):
        raise ValueError("out has the wrong shape")
    code = _dtype_code(q1)
    lib = _lib.load()
    need = int(lib.diffattn_v1_workspace_bytes(B, T, H, d, dv, code))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v1_fwd(
            _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(weight), _ptr(out), B, T, H, d,
            dv, float(lam), float(lambda_init), float(eps), 1 if causal else 0, code,
            _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("diffattn_v1_fwd", rc)
    return out


def _v1_bf16_check(q1, k1, q2, k2, v, weight):
    torch = _torch()
    dev = q1.device
    _check_tensor("q1", q1, dtype=torch.bfloat16, dim=4)
    for n, t in (("k1", k1), ("q2", q2), ("k2", k2)):
        _check_tensor(n, t, dtype=torch.bfloat16, dim=4, device=dev)
        if t.shape != q1.shape:
            raise ValueError(f"{n} shape {tuple(t.shape)} != q1 shape {tuple(q1.shape)}")
    _check_tensor("v", v, dtype=torch.bfloat16, dim=4, device=dev)
    B, T, H, d = q1.shape
    if tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"v shape {tuple(v.shape)} does not match q1 {tuple(q1.shape)}")
    dv = v.shape[3]
    if weight is not None:
        _check_tensor("weight", weight, dtype=torch.float32, dim=1, device=dev)
        if weight.shape[0] != dv:
            raise ValueError("weight must have dv entries")
    return B, T, H, d, dv


def v1_fwd_train(q1, k1, q2, k2, v, lam: float, lambda_init: float, eps: float = 1e-12,
                 weight=None, causal: bool = True, workspace=None, outs=None):
    """DIFF V1 training forward (bf16 inputs).

    Returns (out [B,T,H,dv], o1 [B,T,H,dv], o2 [B,T,H,dv], lse [B,T,H,2]), all
    fp32: o1, o2 are the per-map normalised outputs, lse their log-sum-exp.
    ``outs``: the same four tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q1.device
    B, T, H, d, dv = _v1_bf16_check(q1, k1, q2, k2, v, weight)
    f32 = torch.float32
    out, o1, o2, lse = _outputs("v1_fwd_train", outs, [
        ("out", (B, T, H, dv), f32), ("o1", (B, T, H, dv), f32), ("o2", (B, T, H, dv), f32),
        ("lse", (B, T, H, 2), f32)], dev)
    lib = _lib.load()
    need = int(lib.diffattn_v1_workspace_bytes(B, T, H, d, dv, DIFFATTN_BF16))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v1_fwd_train(
            _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(weight), _ptr(out), _ptr(o1),
            _ptr(o2), _ptr(lse), B, T, H, d, dv, float(lam), float(lambda_init), float(eps),
            1 if causal else 0, DIFFATTN_BF16, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("diffattn_v1_fwd_train", rc)
    return out, o1, o2, lse


def v1_bwd_workspace_bytes(B, T, H, d, dv) -> int:
    return int(_lib.load().diffattn_v1_bwd_workspace_bytes(B, T, H, d, dv))


def v1_bwd(q1, k1, q2, k2, v, o1, o2, lse, dy, lam: float, lambda_init: float,
           eps: float = 1e-12, weight=None, causal: bool = True, workspace=None, outs=None):
    """DIFF V1 backward (bf16 inputs): gradients of sum(dy * y).

    o1, o2, lse from v1_fwd_train on the same inputs; dy [B,T,H,dv] fp32 ->
    (dq1, dk1, dq2, dk2 [B,T,H,d], dv [B,T,H,dv], dlambda [1], dweight [dv]),
    all fp32.  dweight is the gradient of the norm weight (ones when weight is None).
    ``outs``: the same seven tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q1.device
    B, T, H, d, dv = _v1_bf16_check(q1, k1, q2, k2, v, weight)
    for n, t in (("o1", o1), ("o2", o2), ("dy", dy)):
        _check_tensor(n, t, dtype=torch.float32, dim=4, device=dev)
        if tuple(t.shape) != (B, T, H, dv):
            raise ValueError(f"{n} must have shape {(B, T, H, dv)}")
    _check_tensor("lse", lse, dtype=torch.float32, dim=4, device=dev)
    if tuple(lse.shape) != (B, T, H, 2):
        raise ValueError(f"lse must have shape {(B, T, H, 2)}")
    f32 = torch.float32
    dq1, dk1, dq2, dk2, dvv, dlam, dw = _outputs("v1_bwd", outs, [
        ("dq1", (B, T, H, d), f32), ("dk1", (B, T, H, d), f32), ("dq2", (B, T, H, d), f32),
        ("dk2", (B, T, H, d), f32), ("dv", (B, T, H, dv), f32), ("dlambda", (1,), f32),
        ("dweight", (dv,), f32)], dev)
    lib = _lib.load()
    need = int(lib.diffattn_v1_bwd_workspace_bytes(B, T, H, d, dv))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v1_bwd(
            _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(weight), _ptr(o1), _ptr(o2),
            _ptr(lse), _ptr(dy), _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2), _ptr(dvv), _ptr(dlam),
            _ptr(dw), B, T, H, d, dv, float(lam), float(lambda_init), float(eps),
            1 if causal else 0, DIFFATTN_BF16, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("diffattn_v1_bwd", rc)
    return dq1, dk1, dq2, dk2, dvv, dlam, dw


def _signal_heads(Hq: int, ratio: int) -> int:
    """Output heads of blocks of ``ratio`` signal heads and one noise head."""
    if ratio < 1 or Hq % (ratio + 1):
        raise ValueError(f"Hq={Hq} must be a multiple of ratio + 1 = {ratio + 1}")
    return Hq // (ratio + 1) * ratio


def _prefill(fn, ratio, q, k, v, logit, cu_seqlens, max_seqlen, causal, scale, out):
    torch = _torch()
    dev = q.device
    packed = cu_seqlens is not None
    nd = 3 if packed else 4
    _check_tensor("q", q, dtype=torch.bfloat16, dim=nd)
    _check_tensor("k", k, dtype=torch.bfloat16, dim=nd, device=dev)
    _check_tensor("v", v, dtype=torch.bfloat16, dim=nd, device=dev)
    _check_tensor("logit", logit, dtype=torch.float32, dim=nd - 1, device=dev)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    lead = tuple(q.shape[:nd - 2])
    Hq, d = q.shape[-2], q.shape[-1]
    Hkv = k.shape[-2]
    if tuple(k.shape[:nd - 2]) != lead or k.shape[-1] != d:
        raise ValueError("k/v shape does not match q")
    Hs = _signal_heads(Hq, ratio)
    if tuple(logit.shape) != lead + (Hs,):
        raise ValueError(f"logit must have shape {lead + (Hs,)}")
    if out is None:
        out = torch.empty(lead + (Hs, d), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, dtype=torch.bfloat16, dim=nd, device=dev)
    if tuple(out.shape) != lead + (Hs, d):
        raise ValueError("out has the wrong shape")
    if packed:
        _check_tensor("cu_seqlens", cu_seqlens, dtype=torch.int32, dim=1, device=dev)
        if max_seqlen is None:
            raise ValueError("max_seqlen (a host int) is required with cu_seqlens")
        nseq = cu_seqlens.shape[0] - 1
        B, T = 0, lead[0]  # packed: T carries the token count N
    else:
        nseq, max_seqlen = 0, 0
        B, T = lead
    lib = _lib.load()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(out), _ptr(cu_seqlens), nseq,
            int(max_seqlen), B, T, Hq, Hkv, d]
    if fn == "diffattn_gda_fwd":
        args.append(int(ratio))
    with torch.cuda.device(dev):
        rc = getattr(lib, fn)(*args, float(scale or 0.0), 1 if causal else 0, DIFFATTN_BF16,
                              _stream(dev))
    _lib.check(fn, rc)
    return out


def v2_fwd(q, k, v, logit, cu_seqlens=None, max_seqlen=None, causal: bool = True,
           scale: float | None = None, out=None):
    """DIFF V2 forward.

    Padded: q [B,T,Hq,d], k/v [B,T,Hkv,d] bf16, logit [B,T,Hq/2] fp32 -> out [B,T,Hq/2,d] bf16.
    Packed: q [N,Hq,d], k/v [N,Hkv,d], logit [N,Hq/2], cu_seqlens int32 [nseq+1] on the GPU and
    ``max_seqlen`` (host int, >= every sequence length) -> out [N,Hq/2,d].
    """
    return _prefill("diffattn_v2_fwd", 1, q, k, v, logit, cu_seqlens, max_seqlen, causal, scale,
                    out)


def gda_fwd(q, k, v, logit, ratio: int, cu_seqlens=None, max_seqlen=None, causal: bool = True,
            scale: float | None = None, out=None):
    """Grouped differential attention forward: blocks of ``ratio`` signal heads
    and one noise head (ratio 1 is V2).  Shapes as v2_fwd with Hs = Hq/(ratio+1)*ratio
    output heads: logit [..., Hs] fp32 -> out [..., Hs, d] bf16."""
    return _prefill("diffattn_gda_fwd", ratio, q, k, v, logit, cu_seqlens, max_seqlen, causal,
                    scale, out)


def v2_decode_workspace_bytes(B, S_max, Hq, Hkv, d) -> int:
    return int(_lib.load().diffattn_v2_decode_workspace_bytes(B, S_max, Hq, Hkv, d))


def _decode(fn, ratio, q, k_cache, v_cache, logit, cache_len, scale, out, workspace):
    torch = _torch()
    dev = q.device
    _check_tensor("q", q, dtype=torch.bfloat16, dim=3)
    _check_tensor("k_cache", k_cache, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("v_cache", v_cache, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("logit", logit, dtype=torch.float32, dim=2, device=dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    B, Hq, d = q.shape
    _, S_max, Hkv, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d:
        raise ValueError("cache shape does not match q")
    Hs = _signal_heads(Hq, ratio)
    if tuple(logit.shape) != (B, Hs):
        raise ValueError(f"logit must have shape {(B, Hs)}")
    if cache_len is not None:
        _check_tensor("cache_len", cache_len, dtype=torch.int32, dim=1, device=dev)
        if cache_len.shape[0] != B:
            raise ValueError("cache_len must have B entries")
    if out is None:
        out = torch.empty((B, Hs, d), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, dtype=torch.bfloat16, dim=3, device=dev)
    if tuple(out.shape) != (B, Hs, d):
        raise ValueError("out has the wrong shape")
    lib = _lib.load()
    need = int(lib.diffattn_gda_decode_workspace_bytes(B, S_max, Hq, Hkv, d, ratio))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(logit), _ptr(out),
            _ptr(workspace), ws_bytes, B, S_max, Hq, Hkv, d]
    if fn == "diffattn_gda_decode":
        args.append(int(ratio))
    with torch.cuda.device(dev):
        rc = getattr(lib, fn)(*args, float(scale or 0.0), DIFFATTN_BF16, _stream(dev))
    _lib.check(fn, rc)
    return out


def v2_decode(q, k_cache, v_cache, logit, cache_len=None, scale: float | None = None, out=None,
              workspace=None):
    """DIFF V2 decode step.  q [B,Hq,d], caches [B,S_max,Hkv,d] bf16, logit [B,Hq/2] fp32,
    cache_len int32 [B] on the GPU or None -> out [B,Hq/2,d] bf16."""
    return _decode("diffattn_v2_decode", 1, q, k_cache, v_cache, logit, cache_len, scale, out,
                   workspace)


def gda_decode_workspace_bytes(B, S_max, Hq, Hkv, d, ratio) -> int:
    return int(_lib.load().diffattn_gda_decode_workspace_bytes(B, S_max, Hq, Hkv, d, ratio))


def gda_decode(q, k_cache, v_cache, logit, ratio: int, cache_len=None,
               scale: float | None = None, out=None, workspace=None):
    """Grouped differential attention decode step: as v2_decode with blocks of
    ``ratio`` signal heads and one noise head; logit [B,Hs] -> out [B,Hs,d],
    Hs = Hq/(ratio+1)*ratio."""
    return _decode("diffattn_gda_decode", ratio, q, k_cache, v_cache, logit, cache_len, scale,
                   out, workspace)


def v2_decode_noalloc(q, k_cache, v_cache, logit, cache_len=None, scale: float | None = None,
                      out=None):
    """v2_decode with the partial results in the library's own device array (no
    workspace; for callers that cannot allocate).  ``out`` may be preallocated;
    calls that overlap on one GPU race (they share the array)."""
    torch = _torch()
    dev = q.device
    _check_tensor("q", q, dtype=torch.bfloat16, dim=3)
    _check_tensor("k_cache", k_cache, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("v_cache", v_cache, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("logit", logit, dtype=torch.float32, dim=2, device=dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    B, Hq, d = q.shape
    _, S_max, Hkv, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d:
        raise ValueError("cache shape does not match q")
    if Hq % 2 or tuple(logit.shape) != (B, Hq // 2):
        raise ValueError("Hq must be even and logit must have shape [B, Hq/2]")
    if cache_len is not None:
        _check_tensor("cache_len", cache_len, dtype=torch.int32, dim=1, device=dev)
        if cache_len.shape[0] != B:
            raise ValueError("cache_len must have B entries")
    if out is None:
        out = torch.empty((B, Hq // 2, d), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, dtype=torch.bfloat16, dim=3, device=dev)
    if tuple(out.shape) != (B, Hq // 2, d):
        raise ValueError("out has the wrong shape")
    with torch.cuda.device(dev):
        rc = _lib.load().diffattn_v2_decode_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(logit), _ptr(out), B,
            S_max, Hq, Hkv, d, float(scale or 0.0), DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v2_decode_noalloc", rc)
    return out


def _v2_padded_check(q, k, v, logit):
    torch = _torch()
    dev = q.device
    _check_tensor("q", q, dtype=torch.bfloat16, dim=4)
    _check_tensor("k", k, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("v", v, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("logit", logit, dtype=torch.float32, dim=3, device=dev)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, T, Hq, d = q.shape
    if tuple(k.shape[:2]) != (B, T) or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    if Hq % 2:
        raise ValueError("Hq must be even")
    if tuple(logit.shape) != (B, T, Hq // 2):
        raise ValueError(f"logit must have shape {(B, T, Hq // 2)}")
    return B, T, Hq, k.shape[2], d


def v2_fwd_train(q, k, v, logit, causal: bool = True, scale: float | None = None, outs=None):
    """DIFF V2 training forward (padded batch).

    q [B,T,Hq,d], k/v [B,T,Hkv,d] bf16, logit [B,T,Hq/2] fp32 ->
    (out [B,T,Hq/2,d] bf16, o_heads [B,T,Hq,d] bf16, lse [B,T,Hq] fp32).
    ``outs``: the same three tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q.device
    B, T, Hq, Hkv, d = _v2_padded_check(q, k, v, logit)
    out, o_heads, lse = _outputs("v2_fwd_train", outs, [
        ("out", (B, T, Hq // 2, d), torch.bfloat16), ("o_heads", (B, T, Hq, d), torch.bfloat16),
        ("lse", (B, T, Hq), torch.float32)], dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v2_fwd_train(
            _ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(out), _ptr(o_heads), _ptr(lse), B, T, Hq,
            Hkv, d, float(scale or 0.0), 1 if causal else 0, DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v2_fwd_train", rc)
    return out, o_heads, lse


def v2_bwd_workspace_bytes(B, T, Hq, Hkv, d) -> int:
    return int(_lib.load().diffattn_v2_bwd_workspace_bytes(B, T, Hq, Hkv, d))


def v2_bwd(q, k, v, logit, o_heads, lse, dout, causal: bool = True, scale: float | None = None,
           workspace=None, outs=None):
    """DIFF V2 backward (padded batch): gradients of sum(dout * out).

    o_heads, lse from v2_fwd_train on the same inputs; dout [B,T,Hq/2,d] bf16 ->
    (dq [B,T,Hq,d], dk [B,T,Hkv,d], dv [B,T,Hkv,d], dlogit [B,T,Hq/2]), all fp32.
    ``outs``: the same four tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q.device
    B, T, Hq, Hkv, d = _v2_padded_check(q, k, v, logit)
    _check_tensor("o_heads", o_heads, dtype=torch.bfloat16, dim=4, device=dev)
    _check_tensor("lse", lse, dtype=torch.float32, dim=3, device=dev)
    _check_tensor("dout", dout, dtype=torch.bfloat16, dim=4, device=dev)
    if tuple(o_heads.shape) != (B, T, Hq, d) or tuple(lse.shape) != (B, T, Hq):
        raise ValueError("o_heads / lse shapes do not match q")
    if tuple(dout.shape) != (B, T, Hq // 2, d):
        raise ValueError("dout must have shape [B, T, Hq/2, d]")
    f32 = torch.float32
    dq, dk, dv, dlogit = _outputs("v2_bwd", outs, [
        ("dq", (B, T, Hq, d), f32), ("dk", (B, T, Hkv, d), f32), ("dv", (B, T, Hkv, d), f32),
        ("dlogit", (B, T, Hq // 2), f32)], dev)
    lib = _lib.load()
    need = int(lib.diffattn_v2_bwd_workspace_bytes(B, T, Hq, Hkv, d))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v2_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(o_heads), _ptr(lse), _ptr(dout), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dlogit), _ptr(workspace), ws_bytes, B, T, Hq, Hkv, d,
            float(scale or 0.0), 1 if causal else 0, DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v2_bwd", rc)
    return dq, dk, dv, dlogit


def _v2_packed_check(q, k, v, logit, cu_seqlens):
    torch = _torch()
    dev = q.device
    _check_tensor("q", q, dtype=torch.bfloat16, dim=3)
    _check_tensor("k", k, dtype=torch.bfloat16, dim=3, device=dev)
    _check_tensor("v", v, dtype=torch.bfloat16, dim=3, device=dev)
    _check_tensor("logit", logit, dtype=torch.float32, dim=2, device=dev)
    _check_tensor("cu_seqlens", cu_seqlens, dtype=torch.int32, dim=1, device=dev)
    N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != N or k.shape[2] != d:
        raise ValueError("k/v shape does not match q")
    if Hq % 2 or tuple(logit.shape) != (N, Hq // 2):
        raise ValueError(f"logit must have shape {(N, Hq // 2)} and Hq must be even")
    return N, Hq, k.shape[1], d, cu_seqlens.shape[0] - 1


def v2_varlen_fwd_train(q, k, v, logit, cu_seqlens, max_seqlen: int, causal: bool = True,
                        scale: float | None = None, outs=None):
    """DIFF V2 training forward of a packed batch.

    q [N,Hq,d], k/v [N,Hkv,d] bf16, logit [N,Hq/2] fp32, cu_seqlens int32 [nseq+1] ->
    (out [N,Hq/2,d] bf16, o_heads [N,Hq,d] bf16, lse [N,Hq] fp32).
    ``outs``: the same three tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q.device
    N, Hq, Hkv, d, nseq = _v2_packed_check(q, k, v, logit, cu_seqlens)
    out, o_heads, lse = _outputs("v2_varlen_fwd_train", outs, [
        ("out", (N, Hq // 2, d), torch.bfloat16), ("o_heads", (N, Hq, d), torch.bfloat16),
        ("lse", (N, Hq), torch.float32)], dev)
    with torch.cuda.device(dev):
        rc = _lib.load().diffattn_v2_varlen_fwd_train(
            _ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(cu_seqlens), nseq, int(max_seqlen), N,
            _ptr(out), _ptr(o_heads), _ptr(lse), Hq, Hkv, d, float(scale or 0.0),
            1 if causal else 0, DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v2_varlen_fwd_train", rc)
    return out, o_heads, lse


def v2_varlen_bwd(q, k, v, logit, cu_seqlens, o_heads, lse, dout, causal: bool = True,
                  scale: float | None = None, workspace=None, outs=None):
    """DIFF V2 backward of a packed batch: gradients of sum(dout * out).

    o_heads, lse from v2_varlen_fwd_train; dout [N,Hq/2,d] bf16 ->
    (dq [N,Hq,d], dk [N,Hkv,d], dv [N,Hkv,d], dlogit [N,Hq/2]), all fp32.
    ``outs``: the same four tensors, preallocated (optional).
    """
    torch = _torch()
    dev = q.device
    N, Hq, Hkv, d, nseq = _v2_packed_check(q, k, v, logit, cu_seqlens)
    _check_tensor("o_heads", o_heads, dtype=torch.bfloat16, dim=3, device=dev)
    _check_tensor("lse", lse, dtype=torch.float32, dim=2, device=dev)
    _check_tensor("dout", dout, dtype=torch.bfloat16, dim=3, device=dev)
    if tuple(o_heads.shape) != (N, Hq, d) or tuple(lse.shape) != (N, Hq):
        raise ValueError("o_heads / lse shapes do not match q")
    if tuple(dout.shape) != (N, Hq // 2, d):
        raise ValueError("dout must have shape [N, Hq/2, d]")
    f32 = torch.float32
    dq, dk, dv, dlogit = _outputs("v2_varlen_bwd", outs, [
        ("dq", (N, Hq, d), f32), ("dk", (N, Hkv, d), f32), ("dv", (N, Hkv, d), f32),
        ("dlogit", (N, Hq // 2), f32)], dev)
    lib = _lib.load()
    need = int(lib.diffattn_v2_varlen_bwd_workspace_bytes(N, nseq, Hq, Hkv, d))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v2_varlen_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(cu_seqlens), nseq, _ptr(o_heads),
            _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlogit), _ptr(workspace),
            ws_bytes, N, Hq, Hkv, d, float(scale or 0.0), 1 if causal else 0, DIFFATTN_BF16,
            _stream(dev))
    _lib.check("diffattn_v2_varlen_bwd", rc)
    return dq, dk, dv, dlogit


def v1_decode_workspace_bytes(B, S_max, H, d, dv) -> int:
    return int(_lib.load().diffattn_v1_decode_workspace_bytes(B, S_max, H, d, dv))


def v1_decode(q1, q2, k1_cache, k2_cache, v_cache, lam: float, lambda_init: float,
              eps: float = 1e-12, weight=None, cache_len=None, out=None, workspace=None):
    """DIFF V1 decode step.  q1, q2 [B,H,d]; k1/k2 caches [B,S_max,H,d]; v cache
    [B,S_max,H,dv] bf16; cache_len int32 [B] on the GPU or None -> out [B,H,dv] fp32."""
    torch = _torch()
    dev = q1.device
    _check_tensor("q1", q1, dtype=torch.bfloat16, dim=3)
    _check_tensor("q2", q2, dtype=torch.bfloat16, dim=3, device=dev)
    for n, t in (("k1_cache", k1_cache), ("k2_cache", k2_cache), ("v_cache", v_cache)):
        _check_tensor(n, t, dtype=torch.bfloat16, dim=4, device=dev)
    if q2.shape != q1.shape or k2_cache.shape != k1_cache.shape:
        raise ValueError("q2 / k2_cache must match q1 / k1_cache")
    B, H, d = q1.shape
    _, S_max, Hk, dk = k1_cache.shape
    if k1_cache.shape[0] != B or Hk != H or dk != d:
        raise ValueError("k caches do not match q1")
    if tuple(v_cache.shape[:3]) != (B, S_max, H):
        raise ValueError("v_cache does not match the k caches")
    dv = v_cache.shape[3]
    if weight is not None:
        _check_tensor("weight", weight, dtype=torch.float32, dim=1, device=dev)
        if weight.shape[0] != dv:
            raise ValueError("weight must have dv entries")
    if cache_len is not None:
        _check_tensor("cache_len", cache_len, dtype=torch.int32, dim=1, device=dev)
        if cache_len.shape[0] != B:
            raise ValueError("cache_len must have B entries")
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    _check_tensor("out", out, dtype=torch.float32, dim=3, device=dev)
    if tuple(out.shape) != (B, H, dv):
        raise ValueError("out has the wrong shape")
    lib = _lib.load()
    need = int(lib.diffattn_v1_decode_workspace_bytes(B, S_max, H, d, dv))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_tensor("workspace", workspace, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.diffattn_v1_decode(
            _ptr(q1), _ptr(q2), _ptr(k1_cache), _ptr(k2_cache), _ptr(v_cache), _ptr(cache_len),
            _ptr(weight), _ptr(out), _ptr(workspace), ws_bytes, B, S_max, H, d, dv, float(lam),
            float(lambda_init), float(eps), DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v1_decode", rc)
    return out


def v2_lambda_proj(x, w_lambda, out=None):
    """Coefficient logits of V2: x [N, d_model] bf16, w_lambda [h, d_model] bf16 -> [N, h] fp32."""
    torch = _torch()
    dev = x.device
    _check_tensor("x", x, dtype=torch.bfloat16, dim=2)
    _check_tensor("w_lambda", w_lambda, dtype=torch.bfloat16, dim=2, device=dev)
    N, dm = x.shape
    h = w_lambda.shape[0]
    if w_lambda.shape[1] != dm:
        raise ValueError("w_lambda must be [h, d_model]")
    if out is None:
        out = torch.empty((N, h), dtype=torch.float32, device=dev)
    _check_tensor("out", out, dtype=torch.float32, dim=2, device=dev)
    if tuple(out.shape) != (N, h):
        raise ValueError("out has the wrong shape")
    with torch.cuda.device(dev):
        rc = _lib.load().diffattn_v2_lambda_proj(_ptr(x), _ptr(w_lambda), _ptr(out), N, dm, h,
                                                 DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_v2_lambda_proj", rc)
    return out


def out_proj(attn_out, w_o, out=None):
    """Output projection: attn_out [M, K] bf16, w_o [N, K] bf16 -> [M, N] bf16 (fp32 accumulation)."""
    torch = _torch()
    dev = attn_out.device
    _check_tensor("attn_out", attn_out, dtype=torch.bfloat16, dim=2)
    _check_tensor("w_o", w_o, dtype=torch.bfloat16, dim=2, device=dev)
    M, K = attn_out.shape
    N = w_o.shape[0]
    if w_o.shape[1] != K:
        raise ValueError("w_o must be [N, K]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, dtype=torch.bfloat16, dim=2, device=dev)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    with torch.cuda.device(dev):
        rc = _lib.load().diffattn_out_proj(_ptr(attn_out), _ptr(w_o), _ptr(out), M, K, N,
                                           DIFFATTN_BF16, _stream(dev))
    _lib.check("diffattn_out_proj", rc)
    return out
