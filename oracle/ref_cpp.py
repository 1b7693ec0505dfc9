"""ctypes front of the plain C++ oracle (oracle/ref_forward.cpp).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline leg
may use this module. `build()` compiles the library with g++ (no HIP, no BLAS);
`forward_cpp()` runs the whole forward of the C++ oracle on host arrays and reports the
seconds it took (std::chrono::steady_clock inside the library) and the threads it used.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_forward.cpp")
LIB = os.path.join(HERE, "libref_moe.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle/ref_forward.cpp into oracle/libref_moe.so (always recompiles)."""
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    cmd = [cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C++ oracle failed:\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_from_source(src_text: str, out_path: str) -> str:
    """Compile C++ source text (a copy of ref_forward.cpp) into `out_path` (for tests that
    plant a mistake in a copy)."""
    cpp = out_path + ".cpp"
    with open(cpp, "w") as f:
        f.write(src_text)
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    r = subprocess.run([cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", cpp, "-o", out_path],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building a copy of the C++ oracle failed:\n{r.stderr}")
    return out_path


def _bind(lib):
    P, I32 = ctypes.c_void_p, ctypes.c_int
    lib.ref_moe_forward.argtypes = [P, P, I32, P, P, I32, I32, P, P, P, P, I32, I32, I32, P, I32,
                                    I32, P, P, P, P, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int)]
    lib.ref_moe_forward.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None):
    """The built library (built first if missing), or the library at `path`."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        _lib = _bind(lib)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def forward_cpp(inp: dict, tokens: Optional[Sequence[int]] = None, threads: int = 0,
                keep_intermediates: bool = True, lib=None):
    """The C++ oracle's forward on a dict with keys x_fp8, x_sf, topk_idx, topk_weights, w1,
    w1_sf, w2, w2_sf (host arrays). Returns y_bits [n, H], y (fp64 before rounding), h8 and
    h_sf keyed by slot t*k+j (valid slots of the given tokens), seconds, threads."""
    c = lambda a, dt: np.ascontiguousarray(np.asarray(a), dtype=dt)
    x, xsf = c(inp["x_fp8"], np.uint8), c(inp["x_sf"], np.uint8)
    idx, w = c(inp["topk_idx"], np.int32), c(inp["topk_weights"], np.float32)
    w1, w1s, w2, w2s = (c(inp[n], np.uint8) for n in ("w1", "w1_sf", "w2", "w2_sf"))
    T, H = x.shape
    k = idx.shape[1]
    E, twoI, _ = w1.shape
    I = twoI // 2
    toks = np.arange(T, dtype=np.int32) if tokens is None else c(tokens, np.int32)
    n = len(toks)
    y_bits = np.empty((n, H), dtype=np.uint16)
    y = np.empty((n, H), dtype=np.float64)
    h8 = np.zeros((n * k, I), dtype=np.uint8) if keep_intermediates else None
    hsf = np.zeros((n * k, I // 128), dtype=np.uint8) if keep_intermediates else None
    sec = ctypes.c_double(0.0)
    used = ctypes.c_int(0)
    st = (lib or load()).ref_moe_forward(_p(x), _p(xsf), xsf.shape[1], _p(idx), _p(w), T, k, _p(w1), _p(w1s),
                                _p(w2), _p(w2s), E, H, I, _p(toks), n, int(threads), _p(y_bits), _p(y),
                                _p(h8), _p(hsf), ctypes.byref(sec), ctypes.byref(used))
    if st != 0:
        raise RuntimeError(f"C++ oracle failed with status {st}")
    h8d, hsfd = {}, {}
    if keep_intermediates:
        for i, t in enumerate(toks):
            for j in range(k):
                if 0 <= idx[t, j] < E:
                    h8d[int(t) * k + j] = h8[i * k + j]
                    hsfd[int(t) * k + j] = hsf[i * k + j]
    return dict(y_bits=y_bits, y=y, h8=h8d, h_sf=hsfd, seconds=sec.value, threads=used.value,
                tokens=toks)
