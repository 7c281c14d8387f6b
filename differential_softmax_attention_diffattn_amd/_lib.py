"""ctypes loader for ``libdiffattn.so`` (the gfx950 HIP library) and its C signatures.

The library is linked against ``libamdhip64.so.7``.  PyTorch ships its own copy
of that runtime under the same SONAME, so torch is imported first: the dynamic
loader then reuses torch's runtime and the hipStream_t handles torch hands out
belong to the runtime the library launches on.  A second runtime in the process
is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdiffattn.so")

DIFFATTN_F32 = 0
DIFFATTN_BF16 = 1

ERRORS = {
    -1: "DIFFATTN_E_INVALID",
    -2: "DIFFATTN_E_UNSUPPORTED",
    -3: "DIFFATTN_E_ALIGN",
    -4: "DIFFATTN_E_WORKSPACE",
    -5: "DIFFATTN_E_HIP",
}

_c = ctypes
_vp, _sz, _i, _f, _ll = _c.c_void_p, _c.c_size_t, _c.c_int, _c.c_float, _c.c_longlong

SIGNATURES = {
    "diffattn_v1_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                             _i, _vp, _sz, _vp]),
    "diffattn_v1_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "diffattn_v1_fwd_train": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                   _i, _f, _f, _f, _i, _i, _vp, _sz, _vp]),
    "diffattn_v1_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _i, _i, _vp, _sz,
                             _vp]),
    "diffattn_v1_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "diffattn_v2_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                             _vp]),
    "diffattn_gda_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                              _i, _vp]),
    "diffattn_v2_fwd_train": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                   _i, _vp]),
    "diffattn_v2_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i,
                             _i, _i, _i, _i, _f, _i, _i, _vp]),
    "diffattn_v2_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "diffattn_v2_varlen_fwd_train": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _ll, _vp, _vp, _vp, _i,
                                          _i, _i, _f, _i, _i, _vp]),
    "diffattn_v2_varlen_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _sz, _ll, _i, _i, _i, _f, _i, _i, _vp]),
    "diffattn_v2_varlen_bwd_workspace_bytes": (_sz, [_ll, _i, _i, _i, _i]),
    "diffattn_v2_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _i, _f, _i,
                                _vp]),
    "diffattn_v2_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "diffattn_v2_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                        _vp]),
    "diffattn_gda_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _i, _i,
                                 _f, _i, _vp]),
    "diffattn_gda_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "diffattn_v1_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i,
                                _i, _f, _f, _f, _i, _vp]),
    "diffattn_v1_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "diffattn_v2_lambda_proj": (_i, [_vp, _vp, _vp, _ll, _i, _i, _i, _vp]),
    "diffattn_out_proj": (_i, [_vp, _vp, _vp, _ll, _ll, _ll, _i, _vp]),
    "diffattn_lambda_init": (_f, [_i]),
    "diffattn_last_error": (_c.c_char_p, []),
    "diffattn_version": (_i, []),
}

_lock = threading.Lock()
_lib = None


class DiffAttnError(RuntimeError):
    def __init__(self, fn: str, rc: int, msg: str):
        super().__init__(f"{fn} failed with {ERRORS.get(rc, rc)}: {msg}")
        self.rc = rc


def _hip_runtimes_loaded() -> set[str]:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the library (once) and attach the C signatures.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        import torch  # noqa: F401  (see module docstring: torch's HIP runtime must come first)

        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is missing: build it with `python -m differential_softmax_attention_diffattn_amd.build`"
            )
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        runtimes = _hip_runtimes_loaded()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes loaded in one process: {sorted(runtimes)}")
        _lib = lib
        return lib


def check(fn: str, rc: int) -> None:
    if rc != 0:
        msg = load().diffattn_last_error()
        raise DiffAttnError(fn, rc, msg.decode() if msg else "")
