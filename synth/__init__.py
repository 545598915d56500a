"""Seeded synthetic inputs for the routed-expert FFN step.

This package produces input bytes only (hidden states, router weights and bias,
4-bit expert slabs); it contains none of the method's arithmetic.  The CPU oracle
and the GPU path both consume it.  The C source ``synth.c`` documents the slab
byte layout and the counter-based generator (Philox4x32-10 + Box-Muller).

Workload catalogue: the five synthetic configurations of the routed-expert FFN
step (a tiny one-layer case, batch-1 decode resident and streamed, batch-32
decode streamed, and a 2048-token prefill chunk streamed).  Shapes and value
distributions follow the expert-streaming problem statement of the LayerStoRm
README ("TL;DR": full expert set in pinned host RAM, activated experts streamed
per token, GPU memory used as a cache).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "_synth.so")
_lib = None


def build() -> str:
    """Compile synth.c into _synth.so (plain gcc, OpenMP)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, i32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_x_bf16.argtypes = [u64, u32, u32, i64, i64, vp, i32]
        L.synth_router_w.argtypes = [u64, u32, i64, i64, vp, i32]
        L.synth_rank_permutation.argtypes = [u64, u32, i64, vp]
        L.synth_zipf_bias.argtypes = [u64, u32, i64, ctypes.c_double, vp]
        L.synth_matrix_bytes.argtypes = [i64, i64]
        L.synth_matrix_bytes.restype = i64
        L.synth_slab_bytes.argtypes = [i64, i64]
        L.synth_slab_bytes.restype = i64
        L.synth_expert_slab.argtypes = [u64, u32, u32, i64, i64, vp]
        L.synth_expert_slabs.argtypes = [u64, u32, vp, i64, i64, i64, vp, i32]
        L.synth_expert_slabs_fmt.argtypes = [u64, u32, vp, i64, i64, i64, vp, i32, i32]
        L.synth_slab_bytes_fmt.argtypes = [i64, i64, i32]
        L.synth_slab_bytes_fmt.restype = i64
        L.synth_double_to_bf16.argtypes = [ctypes.c_double]
        L.synth_double_to_bf16.restype = ctypes.c_uint16
        L.synth_double_to_fp16.argtypes = [ctypes.c_double]
        L.synth_double_to_fp16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------- configs
@dataclass(frozen=True)
class Config:
    name: str
    layers: int
    tokens: int       # tokens per step (decode batch or prefill chunk)
    hidden: int
    inter: int
    experts: int
    shared: int       # always-on shared experts (0 or 1)
    top_k: int
    cap: float        # fraction of routed experts per layer the HBM cache holds
    bias: str         # "none" | "zipf"
    zipf_s: float
    seed: int
    description: str
    fmt: int = 0      # expert weight format: 0 = 4-bit codes with fp16 scale/min per 32; 1 = MXFP4; 2 = super-blocks
    # distinct expert weight sets: 0 = every layer its own; n > 0: layer l's routed
    # and shared experts hold the weights of layer l % n (the 16-layer configurations'
    # full host pool, 90 GiB, is more than one process may page-lock on the test
    # machine; with 8 weight sets 45 GiB is pinned and every layer still has its own
    # router, inputs, cache slots and misses, so every streamed byte crosses PCIe)
    weight_layers: int = 0

    @property
    def slots(self) -> int:
        """Cache slots per layer: floor(cap * E)."""
        return int(self.cap * self.experts + 1e-9)

    @property
    def streaming(self) -> bool:
        return self.slots < self.experts

    @property
    def slab_bytes(self) -> int:
        return slab_bytes(self.hidden, self.inter, self.fmt)

    def weight_layer(self, layer: int) -> int:
        """Generator layer id of layer `layer`'s expert weights."""
        return layer % self.weight_layers if self.weight_layers else layer

    @property
    def n_weight_sets(self) -> int:
        return min(self.weight_layers, self.layers) if self.weight_layers else self.layers


CONFIGS = {
    "tiny": Config("tiny", 1, 4, 256, 128, 16, 0, 2, 1.0, "none", 0.0, 20261204,
                   "1 layer, H256, 16 experts, I128, top-2, 4 tokens, resident"),
    "decode1": Config("decode1", 8, 1, 4096, 1536, 128, 1, 8, 1.0, "none", 0.0, 20261205,
                      "decode batch 1: 8 layers, H4096, 128 experts + 1 shared, I1536, top-8, resident"),
    "decode1_stream": Config("decode1_stream", 8, 1, 4096, 1536, 128, 1, 8, 0.25, "zipf", 1.1, 20261206,
                             "decode batch 1, cache cap 25% per layer, Zipf(1.1) router bias, streamed misses"),
    "decode32_stream": Config("decode32_stream", 16, 32, 6144, 2048, 256, 1, 8, 0.40, "zipf", 1.1, 20261207,
                              "decode batch 32: 16 layers, H6144, 256 experts + 1 shared, I2048, top-8, "
                              "Zipf(1.1), cap 40%; layers 8-15 reuse the expert weights of layers 0-7",
                              weight_layers=8),
    "prefill2048_stream": Config("prefill2048_stream", 16, 2048, 6144, 2048, 256, 0, 8, 0.40, "none", 0.0,
                                 20261208, "prefill chunk 2048 tokens: 16 layers, H6144, 256 experts, I2048, "
                                 "top-8, uniform routing, cap 40%; layers 8-15 reuse the expert weights of "
                                 "layers 0-7", weight_layers=8),
    "decode1_mx": Config("decode1_mx", 8, 1, 4096, 1536, 128, 1, 8, 1.0, "none", 0.0, 20261210,
                         "decode batch 1 with MXFP4 expert weights: 8 layers, H4096, 128 experts + 1 shared, "
                         "I1536, top-8, resident", 1),
    "decode1_mx_stream": Config("decode1_mx_stream", 8, 1, 4096, 1536, 128, 1, 8, 0.25, "zipf", 1.1, 20261211,
                                "decode batch 1 with MXFP4 expert weights, cache cap 25% per layer, Zipf(1.1) "
                                "router bias, streamed misses", 1),
    "decode1_sb": Config("decode1_sb", 8, 1, 4096, 1536, 128, 1, 8, 1.0, "none", 0.0, 20261212,
                         "decode batch 1 with super-block expert weights: 8 layers, H4096, 128 experts + 1 shared, "
                         "I1536, top-8, resident", 2),
    "decode1_sb_stream": Config("decode1_sb_stream", 8, 1, 4096, 1536, 128, 1, 8, 0.25, "zipf", 1.1, 20261213,
                                "decode batch 1 with super-block expert weights, cache cap 25% per layer, Zipf(1.1) "
                                "router bias, streamed misses", 2),
}
# the 32-token decode and 2048-token prefill configurations with the other weight formats
for _fmt, _tag, _what in ((1, "mx", "MXFP4"), (2, "sb", "super-block")):
    for _base, _seed in (("decode32_stream", 20261214), ("prefill2048_stream", 20261216)):
        _c = CONFIGS[_base]
        _name = _base.replace("_stream", f"_{_tag}_stream")
        CONFIGS[_name] = replace(_c, name=_name, seed=_seed + _fmt - 1, fmt=_fmt,
                                 description=f"{_c.description}; {_what} expert weights")
ORDER = ["tiny", "decode1", "decode1_stream", "decode32_stream", "prefill2048_stream"]


def get(name: str, **overrides) -> Config:
    return replace(CONFIGS[name], **overrides) if overrides else CONFIGS[name]


# --------------------------------------------------------------------------- generators
def matrix_bytes(rows: int, cols: int) -> int:
    """Bytes of a matrix's rows (each row's codes and records padded to 16 bytes)."""
    return int(lib().synth_matrix_bytes(rows, cols))


def slab_bytes(hidden: int, inter: int, fmt: int = 0) -> int:
    return int(lib().synth_slab_bytes_fmt(hidden, inter, fmt))


def philox(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def x_bf16(seed: int, step: int, layer: int, T: int, H: int, threads: int = 0) -> np.ndarray:
    """Hidden states [T, H] as raw bf16 bits (uint16)."""
    out = np.empty((T, H), dtype=np.uint16)
    lib().synth_x_bf16(seed, step, layer, T, H, _ptr(out), threads)
    return out


def router_w(seed: int, layer: int, E: int, H: int, threads: int = 0) -> np.ndarray:
    out = np.empty((E, H), dtype=np.float32)
    lib().synth_router_w(seed, layer, E, H, _ptr(out), threads)
    return out


def rank_permutation(seed: int, layer: int, E: int) -> np.ndarray:
    out = np.empty(E, dtype=np.int32)
    lib().synth_rank_permutation(seed, layer, E, _ptr(out))
    return out


def router_bias(cfg: Config, layer: int):
    """Router bias [E] fp32, or None when the configuration has no bias."""
    if cfg.bias == "none":
        return None
    out = np.empty(cfg.experts, dtype=np.float32)
    lib().synth_zipf_bias(cfg.seed, layer, cfg.experts, cfg.zipf_s, _ptr(out))
    return out


def expert_slab(seed: int, layer: int, expert: int, H: int, I: int, fmt: int = 0) -> np.ndarray:
    out = np.empty(slab_bytes(H, I, fmt), dtype=np.uint8)
    if fmt == 0:
        lib().synth_expert_slab(seed, layer, expert, H, I, _ptr(out))
    else:
        fill_slabs(seed, layer, [expert], H, I, [out.ctypes.data], 1, fmt)
    return out


def fill_slabs(seed: int, layer: int, experts, H: int, I: int, dst_ptrs, threads: int = 0, fmt: int = 0) -> None:
    """Write the slabs of `experts` of `layer` to the host addresses `dst_ptrs`."""
    ex = np.ascontiguousarray(np.asarray(experts, dtype=np.uint32))
    ptrs = np.ascontiguousarray(np.asarray(dst_ptrs, dtype=np.uint64))
    assert ex.shape == ptrs.shape
    lib().synth_expert_slabs_fmt(seed, layer, _ptr(ex), len(ex), H, I, _ptr(ptrs), threads, fmt)


def shared_expert_id(cfg: Config, j: int = 0) -> int:
    """Generator stream id used for shared expert j (distinct from routed ids)."""
    return cfg.experts + j


def double_to_bf16(v: float) -> int:
    return int(lib().synth_double_to_bf16(float(v)))


def double_to_fp16(v: float) -> int:
    return int(lib().synth_double_to_fp16(float(v)))
