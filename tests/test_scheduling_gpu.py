"""GPU parity of the launch shapes that the scheduling rules produce at their
extremes (through the C ABI, against the oracle):

* packed batches of many short sequences (2048 x 32 tokens, the shape of a
  serving prefill batch) and skewed mixes of one long and many short
  sequences: the tile slots and the binary search over cu_seqlens, forward
  and backward;
* decode with one sequence (B = 1, 32768 cached tokens): small batches split
  the cache into short slices to fill the device.
"""
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


def rms(t) -> float:
    return float(t.double().square().mean().sqrt())


def compare(got, ref, rms_v, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    note(f"{what}: max|err|={err:.3e} bound={TOL_BF16 * rms_v:.3e} relL2={rel:.3e}")
    assert err <= TOL_BF16 * rms_v, f"{what}: max|err| {err:.3e}"
    assert rel <= REL_L2_BF16, f"{what}: relative L2 {rel:.3e}"


def compare_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = float(np.max(np.abs(got - ref)))
    bound = 2e-2 * float(np.max(np.abs(ref)))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    note(f"{what}: max|err|={err:.3e} bound={bound:.3e} relL2={rel:.3e}")
    assert err <= bound and rel <= 1e-2, what


@pytest.mark.parametrize("lengths,Hq,Hkv", [
    ((32,) * 2048, 64, 8),                                   # many short sequences
    ((4000,) + (17,) * 300 + (0, 1, 64, 65, 129), 16, 2),    # one long, many short, edges
])
def test_packed_forward_many_sequences(gpu, lengths, Hq, Hkv):
    w = inp.V2_VARLEN.with_shape(lengths=tuple(lengths), Hq=Hq, Hkv=Hkv)
    x = inp.v2_inputs(w)
    N = sum(lengths)
    cu = x["cu_seqlens"].tolist()
    xg = {k: v.to(gpu) for k, v in x.items()}
    out = da.v2_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], cu_seqlens=xg["cu_seqlens"],
                    max_seqlen=max(lengths))
    torch.cuda.synchronize()
    # every token of a sample of sequences: the first, the last, the longest and
    # a spread of others
    nseq = len(lengths)
    seqs = sorted({0, nseq - 1, int(np.argmax(lengths))} | set(range(0, nseq, max(1, nseq // 40))))
    tokens = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    ref = oracle.v2_varlen_forward(x["q"], x["k"], x["v"], x["logit"], x["cu_seqlens"],
                                   tokens=tokens)
    compare(out[torch.from_numpy(tokens).to(gpu)].float().cpu().numpy(), ref, rms(x["v"]),
            f"v2 packed forward nseq={nseq} N={N} ({len(seqs)} sequences checked)")
    # also through the call that does not know N (launch sized by nseq * max_seqlen)
    lib = da._lib.load()
    out2 = torch.empty_like(out)
    Hq, Hkv, d = w.Hq, w.Hkv, w.d
    with torch.cuda.device(gpu):
        rc = lib.diffattn_v2_fwd(xg["q"].data_ptr(), xg["k"].data_ptr(), xg["v"].data_ptr(),
                                 xg["logit"].data_ptr(), out2.data_ptr(),
                                 xg["cu_seqlens"].data_ptr(), nseq, max(lengths), 0, 0, Hq, Hkv,
                                 d, 0.0, 1, da.DIFFATTN_BF16,
                                 torch.cuda.current_stream(gpu).cuda_stream)
    da._lib.check("diffattn_v2_fwd", rc)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_packed_backward_many_short_sequences(gpu):
    lengths = (3, 17, 0, 1, 64, 65) + (9,) * 200 + (130,)
    w = inp.V2_VARLEN.with_shape(Hq=16, Hkv=2, d=128, lengths=lengths)
    x = inp.v2_inputs(w)
    dout = inp.v2_varlen_dout(w)
    xg = {k: v.to(gpu) for k, v in x.items()}
    _, oh, lse = da.v2_varlen_fwd_train(xg["q"], xg["k"], xg["v"], xg["logit"], xg["cu_seqlens"],
                                        max(lengths))
    grads = da.v2_varlen_bwd(xg["q"], xg["k"], xg["v"], xg["logit"], xg["cu_seqlens"], oh, lse,
                             dout.to(gpu))
    torch.cuda.synchronize()
    cu = [int(c) for c in x["cu_seqlens"].tolist()]
    refs = [np.zeros(g.shape) for g in grads]
    for s in range(len(lengths)):
        a, e = cu[s], cu[s + 1]
        if e == a:
            continue
        r = oracle.v2_sequence_backward(x["q"][a:e], x["k"][a:e], x["v"][a:e], x["logit"][a:e],
                                        dout[a:e])
        for i in range(4):
            refs[i][a:e] = r[i]
    for name, g, r in zip(("dq", "dk", "dv", "dlogit"), grads, refs):
        compare_grad(g.cpu().numpy(), r, f"v2 packed backward {len(lengths)} sequences {name}")


def test_decode_single_sequence_full_cache(gpu):
    w = inp.V2_DECODE.with_shape(B=1)
    x = inp.decode_inputs(w)
    out = da.v2_decode(x["q"].to(gpu), x["k_cache"].to(gpu), x["v_cache"].to(gpu),
                       x["logit"].to(gpu))
    torch.cuda.synchronize()
    ref = oracle.v2_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"])
    compare(out.float().cpu().numpy(), ref, rms(x["v_cache"]), "v2 decode B1 S32768")
    w1 = inp.V1_DECODE.with_shape(B=1)
    y = inp.v1_decode_inputs(w1)
    lam = li = oracle.lambda_init(w1.layer)
    out1 = da.v1_decode(*(y[k].to(gpu) for k in ("q1", "q2", "k1_cache", "k2_cache", "v_cache")),
                        lam, li, w1.eps)
    torch.cuda.synchronize()
    ref1 = oracle.v1_decode(y["q1"], y["q2"], y["k1_cache"], y["k2_cache"], y["v_cache"], lam, li,
                            w1.eps)
    compare(out1.cpu().numpy(), ref1, rms(y["v_cache"]), "v1 decode B1 S32768")


@pytest.mark.parametrize("lengths,Hq,Hkv,max_seqlen", [
    ((1, 32, 0, 17, 31, 5, 32, 2) * 40, 64, 8, 32),    # 32-row query tiles: one per sequence
    ((64, 1, 0, 33, 63, 2) * 30, 8, 2, 64),            # 64-row query tiles (two pairs per KV head)
    ((5, 9, 1) * 50, 16, 2, 20),                       # max_seqlen above every length
])
def test_packed_forward_every_sequence_in_one_tile(gpu, lengths, Hq, Hkv, max_seqlen):
    # when max_seqlen fits one query tile the launch has one tile per sequence
    # and no search over cu_seqlens
    w = inp.V2_VARLEN.with_shape(lengths=tuple(lengths), Hq=Hq, Hkv=Hkv)
    x = inp.v2_inputs(w)
    xg = {k: v.to(gpu) for k, v in x.items()}
    out = da.v2_fwd(xg["q"], xg["k"], xg["v"], xg["logit"], cu_seqlens=xg["cu_seqlens"],
                    max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    ref = oracle.v2_varlen_forward(x["q"], x["k"], x["v"], x["logit"], x["cu_seqlens"])
    compare(out.float().cpu().numpy(), ref, rms(x["v"]),
            f"v2 packed one tile per sequence nseq={len(lengths)} Hq={Hq} max_seqlen={max_seqlen}")
