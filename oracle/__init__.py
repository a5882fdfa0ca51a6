"""CPU oracle for the GDN gating + gated delta-rule decode update.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its Python binding
never do, and nothing here imports them.  The arithmetic lives in
``gdn_oracle.c`` (plain double-precision loops); this module only builds it
with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_libs = {}


def build(force: bool = True, src: str = _SRC, out: str = _LIB, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP across independent units only;
    no fused multiply-add contraction, so each step rounds as written).
    ``src``/``out`` let tests compile deliberately broken copies;
    ``sanitize`` builds it with gcc's AddressSanitizer and
    UndefinedBehaviorSanitizer (load it into a process that preloads
    ``sanitizer_runtime()``)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"]
        if sanitize:
            cmd[1:2] = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
                        "-fsanitize=address,undefined"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """gcc's ASan runtime (to preload)."""
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True).stdout.strip()
    if not os.path.isabs(r):
        raise FileNotFoundError("gcc's libasan.so was not found")
    return r


def _load(path: str = _LIB):
    lib = _libs.get(path)
    if lib is None:
        if path == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        f = lib.gdn_oracle_update
        P = ctypes.c_void_p
        f.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        f.restype = ctypes.c_int
        fg = lib.gdn_oracle_gating
        fg.argtypes = [P] * 6 + [ctypes.c_int64, ctypes.c_int]
        fg.restype = ctypes.c_int
        _libs[path] = lib
    return lib


def _ptr(arr: Optional[np.ndarray]):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def update(q, k, v, a, b, A_log, dt_bias, pool, state_idx, cu_seqlens=None,
           tokens_per_seq: int = 1, scale: float = 0.0, eps: float = 1e-6,
           intermediates: bool = False, no_final_writeback: bool = False,
           threads: int = 0, lib_path: str = _LIB, state_layout: str = "KV"):
    """Run the oracle.  ``pool`` (float32 [slots, H_v, K, V], or [slots, H_v,
    V, K] with state_layout "VK"; uint16 bf16 bit patterns for bf16 state
    storage) is updated in place.  Returns ``(out, inter)``: out is float64 [N, H_v, V] (rows of
    untouched tokens stay NaN), inter is float32 [N, H_v, K, V] (NaN where not
    written) or None.  ``lib_path`` selects another build of the same source."""
    lib = _load(lib_path)
    d = np.float64
    q = np.ascontiguousarray(q, dtype=d)
    k = np.ascontiguousarray(k, dtype=d)
    v = np.ascontiguousarray(v, dtype=d)
    a = np.ascontiguousarray(a, dtype=d)
    b = np.ascontiguousarray(b, dtype=d)
    A_log = np.ascontiguousarray(A_log, dtype=d)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=d)
    idx = np.ascontiguousarray(state_idx, dtype=np.int32)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if pool.dtype not in (np.float32, np.uint16) or not pool.flags.c_contiguous:
        raise ValueError("pool must be a C-contiguous float32 or uint16 (bf16) array "
                         "(updated in place)")
    bf16 = pool.dtype == np.uint16
    N, Hk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or a.shape != (N, Hv) or b.shape != (N, Hv):
        raise ValueError("inconsistent activation shapes")
    if state_layout not in ("KV", "VK"):
        raise ValueError("state_layout must be 'KV' or 'VK'")
    tile = (K, V) if state_layout == "KV" else (V, K)
    if pool.shape[1:] != (Hv,) + tile:
        raise ValueError(f"pool shape must be [slots, H_v, {tile[0]}, {tile[1]}]")
    out = np.full((N, Hv, V), np.nan, dtype=d)
    if not intermediates:
        inter = None
    elif bf16:
        inter = np.full((N, Hv) + tile, 0x7fc0, dtype=np.uint16)   # bf16 NaN where not written
    else:
        inter = np.full((N, Hv) + tile, np.nan, dtype=np.float32)
    B = idx.shape[0]
    rc = lib.gdn_oracle_update(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                               _ptr(A_log), _ptr(dt_bias), _ptr(pool), _ptr(idx),
                               _ptr(cu), _ptr(out), _ptr(inter),
                               B, tokens_per_seq, N, Hk, Hv, K, V, pool.shape[0],
                               float(scale), float(eps), int(no_final_writeback),
                               0 if state_layout == "KV" else 1, 1 if bf16 else 0, int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, inter


def gating(a, b, A_log, dt_bias, lib_path: str = _LIB):
    """The standalone gating step: returns (g, beta) as float64 [N, H_v]."""
    lib = _load(lib_path)
    d = np.float64
    a = np.ascontiguousarray(a, dtype=d)
    b = np.ascontiguousarray(b, dtype=d)
    A_log = np.ascontiguousarray(A_log, dtype=d)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=d)
    N, Hv = a.shape
    if b.shape != a.shape or A_log.shape != (Hv,) or dt_bias.shape != (Hv,):
        raise ValueError("inconsistent gate shapes")
    g = np.full((N, Hv), np.nan)
    beta = np.full((N, Hv), np.nan)
    rc = lib.gdn_oracle_gating(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta),
                               N, Hv)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return g, beta


def run_inputs(inp, pool: np.ndarray, scale: float = 0.0, eps: float = 1e-6,
               intermediates: Optional[bool] = None, no_final_writeback=False,
               threads: int = 0, state_layout: str = "KV"):
    """Run the oracle on a ``workloads.HostInputs`` bundle."""
    wl = inp.wl
    if intermediates is None:
        intermediates = wl.intermediates
    return update(inp.q, inp.k, inp.v, inp.a, inp.b, inp.A_log, inp.dt_bias,
                  pool, inp.state_idx, inp.cu_seqlens,
                  tokens_per_seq=wl.tokens_per_seq, scale=scale, eps=eps,
                  intermediates=intermediates,
                  no_final_writeback=no_final_writeback, threads=threads,
                  state_layout=state_layout)
