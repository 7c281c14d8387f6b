"""The V2 decode entry point that allocates nothing (diffattn_v2_decode_noalloc,
for callers that cannot allocate), through the C ABI: its output equals the
workspace entry point's on the same inputs, bit for bit (same kernels and
split), on two calls in a row, the second with a smaller input; sizes beyond
its array are rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import differential_softmax_attention_diffattn_amd as da
from differential_softmax_attention_diffattn_amd import _lib
from differential_softmax_attention_diffattn_amd import inputs as inp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: this test needs an MI355X")
    torch.cuda.init()
    return torch.device("cuda:0")


def test_noalloc_decode_matches_workspace_decode(gpu):
    cases = [inp.V2_DECODE.with_shape(B=6, S=5000, Hq=16, Hkv=2, cache_lens=(5000, 1, 0, 2500, 77, 4999)),
             inp.V2_DECODE.with_shape(B=2, S=700, Hq=16, Hkv=2, cache_lens=(700, 33))]
    for w in cases:
        x = {k: (None if v is None else v.to(gpu)) for k, v in inp.decode_inputs(w).items()}
        ref = da.v2_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"], cache_len=x["cache_len"])
        got = da.v2_decode_noalloc(x["q"], x["k_cache"], x["v_cache"], x["logit"],
                                   cache_len=x["cache_len"])
        torch.cuda.synchronize()
        print(f"noalloc decode B={w.B} S={w.S}: max|diff| = "
              f"{float((got.float() - ref.float()).abs().max()):.3e}", flush=True)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref)


def test_noalloc_decode_rejects_sizes_beyond_its_array(gpu):
    lib = _lib.load()
    limit = 32 << 20
    B, S, Hq, Hkv, d = 2048, 4096, 64, 8, 128
    assert lib.diffattn_v2_decode_workspace_bytes(B, S, Hq, Hkv, d) > limit
    p = 1 << 20  # never dereferenced: rejected before any launch
    rc = lib.diffattn_v2_decode_noalloc(p, p, p, None, p, p, B, S, Hq, Hkv, d, 0.0,
                                        da.DIFFATTN_BF16, None)
    assert rc == -2  # DIFFATTN_E_UNSUPPORTED
    assert b"array" in lib.diffattn_last_error()
