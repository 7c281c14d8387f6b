"""HIP graph capture of the library's calls through the C ABI.

The entry points allocate nothing, synchronise nothing and take every buffer
(outputs and workspaces) from the caller, so a sequence of calls captured on a
stream (torch.cuda.CUDAGraph) replays to the eager results.  One graph holds a
V2 prefill, a V2 training forward and backward, a V2 decode step (split and
combine kernels) and a V1 forward (V pack and fused kernel).  Every replay is
compared bit for bit with eager calls on the same inputs (the kernels are
deterministic); between replays the inputs are rewritten in place and other
eager work runs on the device, and each replay must follow the new inputs.
"""
import sys

import pytest
import torch

import differential_softmax_attention_diffattn_amd as da
from differential_softmax_attention_diffattn_amd import inputs as inp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: these tests need an MI355X")
    torch.cuda.init()
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_graph_replays_match_eager_calls(gpu):
    w2 = inp.V2_PREFILL.with_shape(B=1, T=300, Hq=16, Hkv=2)
    wd = inp.V2_DECODE.with_shape(B=2, S=700, Hq=16, Hkv=2, cache_lens=(700, 333))
    w1 = inp.V1_BF16.with_shape(B=1, T=200, H=2)
    lam = da.lambda_init(3)

    def draw(shift):
        # inputs of the three workloads; the shift moves every seed
        sh = lambda w: w.with_shape(seeds=tuple(s + shift for s in w.seeds))
        x2 = inp.v2_inputs(sh(w2), device=gpu)
        dout = inp.v2_dout(w2, seed=inp.DOUT_SEED + shift, device=gpu)
        xd = inp.decode_inputs(sh(wd), device=gpu)
        x1 = inp.v1_inputs(sh(w1), device=gpu)
        return x2, dout, xd, x1

    x2, dout, xd, x1 = draw(0)  # the static inputs the graph reads
    B, T, Hq, Hkv, d = w2.B, w2.T, w2.Hq, w2.Hkv, w2.d
    ws_b = torch.empty(da.v2_bwd_workspace_bytes(B, T, Hq, Hkv, d), dtype=torch.uint8, device=gpu)
    ws_d = torch.empty(da.v2_decode_workspace_bytes(wd.B, wd.S, wd.Hq, wd.Hkv, wd.d),
                       dtype=torch.uint8, device=gpu)
    ws_1 = torch.empty(max(1, da.v1_workspace_bytes(w1.B, w1.T, w1.H, w1.d, w1.dv, torch.bfloat16)),
                       dtype=torch.uint8, device=gpu)

    def alloc():
        bf, f32 = torch.bfloat16, torch.float32
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=gpu)
        return {
            "v2": z((B, T, Hq // 2, d), bf),
            "t_out": z((B, T, Hq // 2, d), bf), "oh": z((B, T, Hq, d), bf), "lse": z((B, T, Hq), f32),
            "dq": z((B, T, Hq, d), f32), "dk": z((B, T, Hkv, d), f32), "dv": z((B, T, Hkv, d), f32),
            "dlogit": z((B, T, Hq // 2), f32),
            "dec": z((wd.B, wd.Hq // 2, wd.d), bf),
            "v1": z((w1.B, w1.T, w1.H, w1.dv), f32),
        }

    def run(o):
        da.v2_fwd(x2["q"], x2["k"], x2["v"], x2["logit"], out=o["v2"])
        da.v2_fwd_train(x2["q"], x2["k"], x2["v"], x2["logit"], outs=(o["t_out"], o["oh"], o["lse"]))
        da.v2_bwd(x2["q"], x2["k"], x2["v"], x2["logit"], o["oh"], o["lse"], dout, workspace=ws_b,
                  outs=(o["dq"], o["dk"], o["dv"], o["dlogit"]))
        da.v2_decode(xd["q"], xd["k_cache"], xd["v_cache"], xd["logit"], cache_len=xd["cache_len"],
                     out=o["dec"], workspace=ws_d)
        da.v1_fwd(x1["q1"], x1["k1"], x1["q2"], x1["k2"], x1["v"], lam, lam, w1.eps, out=o["v1"],
                  workspace=ws_1)

    eager, graphed = alloc(), alloc()
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(graphed)
    torch.cuda.synchronize()

    other = alloc()
    for rep in range(4):
        if rep > 0:  # new input values, written in place into the tensors the graph reads
            n2, nd, ndd, n1 = draw(rep)
            for old, new in ((x2, n2), (xd, ndd), (x1, n1)):
                for k, t in old.items():
                    if t is not None:
                        t.copy_(new[k])
            dout.copy_(nd)
            torch.cuda.synchronize()
        note(f"graph replay {rep}")
        for t in graphed.values():
            t.fill_(float("nan") if t.dtype.is_floating_point else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(eager)  # the same calls, eagerly, on the same inputs
        torch.cuda.synchronize()
        for name in eager:
            assert torch.equal(graphed[name], eager[name]), f"replay {rep}: {name} differs from eager"
        run(other)  # unrelated eager work between replays
        torch.cuda.synchronize()
    note("graph replays match the eager calls")
