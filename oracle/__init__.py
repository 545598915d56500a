"""CPU oracle for the routed-expert FFN step (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may use this package; the GPU library and its binding never do.
It shares no code with the GPU path.  ``oracle.c`` states what it computes and
which passage each step follows.

Parity status per function (what pins it, see tests/test_oracle_pins.py):
  router logits  -- exact rational sum rounded once to fp32 (brute force, tiny H)
  top-k          -- rank counting brute force; crafted exact ties; all-zero router
  weights        -- k=1 gives 1, equal logits give 1/k, k=E equals scipy softmax
  dequant        -- hand-built slabs with known codes/scales (round trip)
  gate/up, down  -- one-hot inputs recover hand-built columns (layout, nibbles)
  SwiGLU         -- closed-form points (silu(0)=0, g=2,u=3) with gate/up distinct
  expert FFN     -- constant-code experts give a closed form for y
  combine        -- zero routed experts leave the shared expert; k=1 gives y;
                    expert relabelling leaves the output unchanged
  residual norm  -- a constant row normalises to +-1; a row that is sqrt(H) times
                    a unit vector is returned unchanged; positive scaling leaves
                    the output unchanged; the fp32 update equals numpy's fp32 add
The end-to-end values on random inputs have no printed worked example to pin
them; they rest on the pins above.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# MOE_ORACLE_LIB: load another build of oracle.c (the pin-strength test loads
# copies with a planted mistake this way)
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "_oracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c (gcc, -O2, no fast-math, no FMA contraction, OpenMP)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
                           "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_fp16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_fp16_to_double.restype = ctypes.c_double
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_slab_bytes.argtypes = [i64, i64]
        L.oracle_slab_bytes.restype = i64
        L.oracle_dequant.argtypes = [vp, i64, i64, i32, vp]
        L.oracle_expert_ffn.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.oracle_expert_down.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_router.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp, vp, vp, i32]
        L.oracle_moe_layer.argtypes = [vp, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, i64, i32,
                                       vp, vp, vp, vp]
        L.oracle_residual_norm.argtypes = [vp, vp, i64, i64, ctypes.c_double, vp]
        L.oracle_slab_bytes_fmt.argtypes = [i64, i64, i32]
        L.oracle_slab_bytes_fmt.restype = i64
        L.oracle_e2m1_to_double.argtypes = [i32]
        L.oracle_e2m1_to_double.restype = ctypes.c_double
        L.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_to_double.restype = ctypes.c_double
        L.oracle_dequant_fmt.argtypes = [vp, i64, i64, i32, vp, i32]
        L.oracle_expert_ffn_fmt.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, i32]
        L.oracle_moe_layer_fmt.argtypes = [vp, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, i64, i32,
                                           vp, vp, vp, vp, i32]
        L.oracle_moe_ffn_routed_fmt.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, i64, i32, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def fp16_to_double(h: int) -> float:
    return lib().oracle_fp16_to_double(int(h))


def double_to_bf16(v: float) -> int:
    return int(lib().oracle_double_to_bf16(float(v)))


def slab_bytes(H: int, I: int, fmt: int = 0) -> int:
    return int(lib().oracle_slab_bytes_fmt(H, I, fmt))


def e2m1_to_double(q: int) -> float:
    return lib().oracle_e2m1_to_double(q)


def e8m0_to_double(v: int) -> float:
    return lib().oracle_e8m0_to_double(v)


def dequant(slab: np.ndarray, H: int, I: int, which: int, fmt: int = 0) -> np.ndarray:
    rows, cols = (I, H) if which < 2 else (H, I)
    out = np.empty((rows, cols), dtype=np.float64)
    lib().oracle_dequant_fmt(_p(slab), H, I, which, _p(out), fmt)
    return out


def expert_ffn(slab: np.ndarray, H: int, I: int, x: np.ndarray, fmt: int = 0):
    """One token (x: float64 [H]) through one expert -> (g, u, h, y)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    g, u, h = (np.empty(I, np.float64) for _ in range(3))
    y = np.empty(H, np.float64)
    lib().oracle_expert_ffn_fmt(_p(slab), H, I, _p(x), _p(g), _p(u), _p(h), _p(y), fmt)
    return g, u, h, y


def expert_down(slab: np.ndarray, H: int, I: int, h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float64)
    y = np.empty(H, np.float64)
    lib().oracle_expert_down(_p(slab), H, I, _p(h), _p(y))
    return y


def router(x_bf16: np.ndarray, Wr: np.ndarray, bias, k: int, threads: int = 0):
    """-> (logits fp32 [T,E], idx int32 [T,k], w fp64 [T,k])."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    assert Wr.shape[1] == H
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    logits = np.empty((T, E), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_router(_p(x_bf16), T, H, _p(Wr), _p(b), E, k, _p(logits), _p(idx), _p(w), threads)
    return logits, idx, w


def moe_layer(x_bf16: np.ndarray, Wr: np.ndarray, bias, k: int, slabs, shared, I: int,
              rows=None, threads: int = 0, fmt: int = 0):
    """One MoE layer.  slabs: list of E uint8 arrays; shared: uint8 array or None.

    rows: optional list of token indices to compute (others are left zero).
    Returns dict(idx, w, out64 [T,H] float64, out_bf16 [T,H] uint16).
    """
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    assert len(slabs) == E
    sb = slab_bytes(H, I, fmt)
    for s in slabs:
        assert s.dtype == np.uint8 and s.size == sb and s.flags["C_CONTIGUOUS"]
    ptrs = np.array([s.ctypes.data for s in slabs], dtype=np.uint64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    nr = 0 if r is None else len(r)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    out64 = np.zeros((T, H), np.float64)
    outb = np.zeros((T, H), np.uint16)
    lib().oracle_moe_layer_fmt(_p(x_bf16), T, H, I, E, k, _p(Wr), _p(b), _p(ptrs),
                               None if shared is None else _p(shared), _p(r), nr, threads,
                               _p(idx), _p(w), _p(out64), _p(outb), fmt)
    return {"idx": idx, "w": w, "out64": out64, "out_bf16": outb}


def moe_ffn_routed(x_bf16: np.ndarray, idx: np.ndarray, w: np.ndarray, slabs, shared, I: int,
                   rows=None, threads: int = 0, fmt: int = 0):
    """Expert FFNs and the combine for a given routing (steps 4-5 of oracle.c):
    idx [T,k] expert ids, w [T,k] gate weights (taken as given, in fp64).
    Returns dict(out64 [T,H] float64, out_bf16 [T,H] uint16); rows as moe_layer."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H = x_bf16.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    assert idx.shape == w.shape and idx.shape[0] == T
    k = idx.shape[1]
    E = len(slabs)
    assert idx.min() >= 0 and idx.max() < E
    sb = slab_bytes(H, I, fmt)
    for s in slabs:
        assert s.dtype == np.uint8 and s.size == sb and s.flags["C_CONTIGUOUS"]
    ptrs = np.array([s.ctypes.data for s in slabs], dtype=np.uint64)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    nr = 0 if r is None else len(r)
    out64 = np.zeros((T, H), np.float64)
    outb = np.zeros((T, H), np.uint16)
    lib().oracle_moe_ffn_routed_fmt(_p(x_bf16), T, H, I, k, _p(idx), _p(w), _p(ptrs),
                                    None if shared is None else _p(shared), _p(r), nr, threads,
                                    _p(out64), _p(outb), fmt)
    return {"out64": out64, "out_bf16": outb}


def residual_norm(add, resid: np.ndarray, eps: float):
    """Residual update and RMS normalisation of chained layers (see oracle.c).

    add: [T,H] bf16 bits (uint16) or None; resid: [T,H] float32, updated in place.
    Returns x_next [T,H] bf16 bits.
    """
    assert resid.dtype == np.float32 and resid.flags["C_CONTIGUOUS"]
    T, H = resid.shape
    a = None if add is None else np.ascontiguousarray(add, dtype=np.uint16)
    out = np.empty((T, H), np.uint16)
    lib().oracle_residual_norm(_p(a), _p(resid), T, H, ctypes.c_double(eps), _p(out))
    return out
