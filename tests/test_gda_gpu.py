"""GPU parity of grouped differential attention (blocks of `ratio` signal heads
and one noise head inside a GQA group) through the C ABI, against the oracle's
gda_* functions.

Bounds as the V2 tests: max|err| <= 2e-2 * RMS(V) and relative L2 <= 1e-2.
Small cases run every row (ratios 1, 2, 3, 4 and 7; blocks of one, two and
several per group; ragged tails; causal and not; d 64 and 128); the full-size
workloads run as the benchmark launches them and are checked on sampled rows.
Needle keys make single heads' outputs large, so a signal or noise head taken
from the wrong block shows at once.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import differential_softmax_attention_diffattn_amd as da
from differential_softmax_attention_diffattn_amd import inputs as inp

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
REL_L2_BF16 = 1e-2


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: these tests need an MI355X")
    torch.cuda.init()
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rms(t) -> float:
    return float(t.detach().double().square().mean().sqrt().item())


def compare(got, ref, rms_v, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref)))
    bound = TOL_BF16 * rms_v
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    note(f"{what}: max|err|={err:.3e} bound={bound:.3e} ({err / bound:.3f}x) relL2={rel:.3e}")
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e}"
    assert rel <= REL_L2_BF16, f"{what}: relative L2 {rel:.3e}"


def on(x, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in x.items()}


# (Hq, Hkv, ratio): blocks per GQA group 2, 1, 2, 1, 4, 1, 2; output heads per
# group 6, 3, 8, 4, 4, 7, 4 (so one, two and four output heads share a
# workgroup).  Ratios 3 and 7 take the path that attends every head once and
# shares the noise head on chip; 2 and 4 recompute it per signal head.
SHAPES = [(16, 2, 3), (12, 3, 3), (20, 2, 4), (10, 2, 4), (16, 2, 1), (16, 2, 7), (12, 2, 2)]


@pytest.mark.parametrize("Hq,Hkv,ratio", SHAPES)
@pytest.mark.parametrize("d,T,causal", [(128, 200, True), (64, 161, True), (128, 150, False)])
def test_gda_small_all_rows(gpu, Hq, Hkv, ratio, d, T, causal):
    w = inp.V2_PREFILL.with_shape(B=2, T=T, Hq=Hq, Hkv=Hkv, d=d, causal=causal, ratio=ratio)
    x = inp.v2_inputs(w)
    note(f"gda Hq={Hq} Hkv={Hkv} ratio={ratio} d={d} T={T} causal={causal}")
    ref = oracle.gda_forward(x["q"], x["k"], x["v"], x["logit"], ratio, causal=causal)
    xg = on(x, gpu)
    out = da.gda_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], ratio, causal=causal)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), ref, rms(x["v"]),
            f"gda Hq={Hq} Hkv={Hkv} r={ratio} d={d} T={T} causal={causal}")


def test_gda_ratio_one_is_v2_bit_for_bit(gpu):
    w = inp.V2_PREFILL.with_shape(B=2, T=333, Hq=16, Hkv=2)
    xg = on(inp.v2_inputs(w), gpu)
    a = da.gda_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], 1)
    b = da.v2_fwd(xg["q"], xg["k"], xg["v"], xg["logit"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("Hq,Hkv,ratio", [(16, 2, 3), (20, 2, 4)])
def test_gda_packed(gpu, Hq, Hkv, ratio):
    lengths = (37, 64, 0, 130, 5, 1, 257)
    w = inp.V2_VARLEN.with_shape(Hq=Hq, Hkv=Hkv, lengths=lengths, ratio=ratio)
    x = inp.v2_inputs(w)
    cu = x["cu_seqlens"].tolist()
    xg = on(x, gpu)
    note(f"gda packed Hq={Hq} Hkv={Hkv} ratio={ratio} lengths={lengths}")
    out = da.gda_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], ratio,
                     cu_seqlens=xg["cu_seqlens"], max_seqlen=max(lengths))
    torch.cuda.synchronize()
    ref = np.zeros(tuple(out.shape))
    for s in range(len(lengths)):
        a, e = cu[s], cu[s + 1]
        if e > a:
            ref[a:e] = oracle.gda_sequence(x["q"][a:e], x["k"][a:e], x["v"][a:e],
                                           x["logit"][a:e], ratio)
    compare(out.float().cpu().numpy(), ref, rms(x["v"]), f"gda packed r={ratio}")


def test_gda_non_default_scale(gpu):
    w = inp.V2_PREFILL.with_shape(B=1, T=190, Hq=16, Hkv=2, ratio=3)
    x = inp.v2_inputs(w)
    ref = oracle.gda_forward(x["q"], x["k"], x["v"], x["logit"], 3, scale=0.3)
    xg = on(x, gpu)
    out = da.gda_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], 3, scale=0.3)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), ref, rms(x["v"]), "gda scale 0.3")


@pytest.mark.parametrize("Hq,Hkv,ratio,heads", [
    (20, 2, 4, (0, 4, 5, 9, 13, 14, 19)),       # per-signal-head recompute
    (16, 2, 3, (0, 3, 5, 7, 10, 11, 15)),       # noise heads shared on chip
])
def test_gda_needle_heads(gpu, Hq, Hkv, ratio, heads):
    # one needle key per chosen query head: that head's output becomes ~v of
    # the needle, so each output head's result names the signal and noise
    # heads it used
    w = inp.V2_PREFILL.with_shape(B=1, T=256, Hq=Hq, Hkv=Hkv, ratio=ratio)
    x = inp.v2_inputs(w)
    g = w.Hq // w.Hkv
    row = 255
    for n, j in enumerate(heads):
        x["k"][0, 10 * (n + 1), j // g] = (300.0 * x["q"][0, row, j].float()).to(torch.bfloat16)
    ref = oracle.gda_forward(x["q"], x["k"], x["v"], x["logit"], ratio)
    xg = on(x, gpu)
    out = da.gda_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], ratio)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), ref, rms(x["v"]), f"gda needles r={ratio}")


@pytest.mark.parametrize("w", [inp.GDA_PREFILL_R3, inp.GDA_PREFILL_R4], ids=lambda w: w.name)
def test_gda_full_workload_sampled_rows(gpu, w):
    note(f"generating {w.name} on the GPU")
    x = inp.v2_inputs(w, device=gpu)
    out = da.gda_fwd(x["q"], x["k"], x["v"], x["logit"], w.ratio)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 63, 64, 4095, 4096, 8191])
    rv = rms(x["v"])
    for b in range(w.B):
        sl = {k: x[k][b:b + 1].cpu() for k in ("q", "k", "v", "logit")}
        ref = oracle.gda_forward(sl["q"], sl["k"], sl["v"], sl["logit"], w.ratio, rows=rows)
        compare(out[b:b + 1, rows].float().cpu().numpy(), ref, rv, f"{w.name} b={b}")


@pytest.mark.parametrize("B,S,Hq,Hkv,ratio,lens", [(4, 1000, 16, 2, 3, (1000, 1, 0, 517)),
                                                   (2, 5000, 20, 2, 4, (4999, 2048)),
                                                   (3, 700, 12, 3, 3, None)])
def test_gda_decode_small(gpu, B, S, Hq, Hkv, ratio, lens):
    w = inp.V2_DECODE.with_shape(B=B, S=S, Hq=Hq, Hkv=Hkv, d=128, cache_lens=lens, ratio=ratio)
    x = inp.decode_inputs(w)
    g = Hq // Hkv
    # needles: a few heads of entry 0 attend to one key each
    for j, s_ in ((0, 5), (ratio, 100), (ratio + 1, 300), (Hq - 1, 600)):
        x["k_cache"][0, s_, j // g] = (400.0 * x["q"][0, j].float()).to(torch.bfloat16)
    ref = oracle.gda_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"], ratio,
                            cache_len=None if lens is None else np.array(lens))
    xg = on(x, gpu)
    out = da.gda_decode(xg["q"], xg["k_cache"], xg["v_cache"], xg["logit"], ratio,
                        cache_len=xg["cache_len"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    compare(got, ref, rms(x["v_cache"]), f"gda decode B={B} S={S} Hq={Hq} r={ratio}")
    if lens is not None:
        for b, n in enumerate(lens):
            if n == 0:
                assert np.all(got[b] == 0.0)


def test_gda_decode_ratio_one_is_v2_bit_for_bit(gpu):
    w = inp.V2_DECODE.with_shape(B=3, S=900, Hq=16, Hkv=2, cache_lens=(900, 17, 0))
    xg = on(inp.decode_inputs(w), gpu)
    a = da.gda_decode(xg["q"], xg["k_cache"], xg["v_cache"], xg["logit"], 1,
                      cache_len=xg["cache_len"])
    b = da.v2_decode(xg["q"], xg["k_cache"], xg["v_cache"], xg["logit"], cache_len=xg["cache_len"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gda_decode_full_workload_sampled_entries(gpu):
    w = inp.GDA_DECODE_R3
    note(f"generating {w.name} on the GPU")
    x = inp.decode_inputs(w, device=gpu)
    out = da.gda_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"], w.ratio)
    torch.cuda.synchronize()
    for b in (0, 31, 63):
        ref = oracle.gda_decode(x["q"][b:b + 1].cpu(), x["k_cache"][b:b + 1].cpu(),
                                x["v_cache"][b:b + 1].cpu(), x["logit"][b:b + 1].cpu(), w.ratio)
        compare(out[b:b + 1].float().cpu().numpy(), ref, rms(x["v_cache"][b]),
                f"{w.name} b={b}")
