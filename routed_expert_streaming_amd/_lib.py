"""ctypes binding of libmoe.so: the C ABI declared in include/moe.h, same names.

Argument marshalling only: pointers may be given as ints or as objects with a
``data_ptr()`` method (torch tensors); streams as ints, torch streams or None.
A non-zero status raises MoEError carrying the library's message.  Nothing
here computes any part of the method, and nothing falls back to the CPU: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_E_ARG, MOE_E_SHAPE, MOE_E_NOT_PINNED, MOE_E_NOMEM, MOE_E_CAPACITY, MOE_E_HIP, MOE_E_STATE = \
    0, -1, -2, -3, -4, -5, -6, -7
MOE_FFN_AUTO, MOE_FFN_PAIRS, MOE_FFN_GROUPED, MOE_FFN_MFMA, MOE_FFN_SPLIT = 0, 1, 2, 3, 4

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status} ({message})")
        self.status = status


class moe_cache_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("n_experts", ctypes.c_int), ("hidden", ctypes.c_int),
                ("inter", ctypes.c_int), ("slots_per_layer", ctypes.c_int), ("format", ctypes.c_int)]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(MOE_E_STATE, "load", f"{LIB_PATH} is not built; run "
                           "`python -m routed_expert_streaming_amd.build`")
        # torch carries its own HIP runtime (soname libamdhip64.so.7).  Loading it
        # first makes libmoe.so bind to that same runtime, so the streams and device
        # pointers torch hands out are valid for this library.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        _check_single_hip_runtime()
        vp, i, sz, u64p = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint64)
        sig = {
            "moe_status_str": ([i], ctypes.c_char_p),
            "moe_last_hip_error": ([], i),
            "moe_last_error_message": ([], ctypes.c_char_p),
            "moe_version": ([], i),
            "moe_expert_bytes": ([i, i], sz),
            "moe_router_workspace_bytes": ([i, i], sz),
            "moe_router_topk": ([vp, i, i, vp, vp, i, i, vp, vp, vp, sz, vp], i),
            "moe_router_layers_workspace_bytes": ([i, i, i], sz),
            "moe_router_topk_layers": ([vp, i, i, i, vp, vp, i, i, vp, vp, vp, sz, vp], i),
            "moe_permute": ([vp, i, i, i, vp, vp, vp, vp], i),
            "moe_cache_create": ([ctypes.POINTER(moe_cache_desc), vp, vp, vp, vp, ctypes.POINTER(vp)], i),
            "moe_cache_create_recording": ([ctypes.POINTER(moe_cache_desc), ctypes.c_uint64, i,
                                            ctypes.POINTER(vp)], i),
            "moe_cache_trace": ([vp, vp, ctypes.c_int64], ctypes.c_int64),
            "moe_cache_lookup": ([vp, i, vp, i, vp, ctypes.POINTER(i)], i),
            "moe_cache_prefetch": ([vp, i, vp, i, vp, ctypes.POINTER(i)], i),
            "moe_cache_prefetch_async": ([vp, i, vp, i, ctypes.POINTER(i)], i),
            "moe_cache_wait": ([vp, i, vp], i),
            "moe_cache_split_copies": ([vp, vp], i),
            "moe_cache_release": ([vp, i, vp], i),
            "moe_cache_stats": ([vp, u64p, u64p, u64p], i),
            "moe_cache_reset": ([vp], i),
            "moe_cache_copy_timing": ([vp, i], i),
            "moe_cache_copy_busy": ([vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), u64p], i),
            "moe_cache_plan": ([vp, i, vp, i, vp, vp, i, vp, ctypes.POINTER(i)], i),
            "moe_cache_plan_step": ([vp, vp, i, vp, vp, i, vp, vp, i, ctypes.POINTER(i)], i),
            "moe_cache_destroy": ([vp], None),
            "moe_expert_ffn_workspace_bytes": ([i, i, i, i, i, i], sz),
            "moe_expert_ffn": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, sz, i, vp], i),
            "moe_expert_gate_up": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, vp, vp, i, vp], i),
            "moe_expert_ffn_fmt": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, sz, i, i, vp], i),
            "moe_expert_gate_up_fmt": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, vp], i),
            "moe_expert_down_fmt": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, vp], i),
            "moe_quant_act_mx": ([vp, i, i, vp, vp, vp], i),
            "moe_expert_down": ([vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, vp, vp, i, vp], i),
            "moe_expert_ffn_combine": ([vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, sz, i, vp], i),
            "moe_route_ffn_combine_workspace_bytes": ([i, i, i, i, i, i], sz),
            "moe_route_ffn_combine": ([vp, i, i, i, vp, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp], i),
            "moe_combine": ([vp, vp, i, i, i, i, vp, vp], i),
            "moe_scatter_rows": ([vp, vp, i, i, vp, vp], i),
            "moe_noalloc_scratch_bytes": ([], sz),
            "moe_route_ffn_combine_noalloc": ([vp, i, i, i, vp, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp], i),
            "moe_residual_norm": ([vp, vp, i, i, ctypes.c_float, vp, vp], i),
            "moe_debug_dequant": ([vp, i, i, i, vp, vp], i),
            "moe_expert_bytes_mx": ([i, i], sz),
            "moe_expert_bytes_sb": ([i, i], sz),
            "moe_sb_expert_ffn_combine": ([vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, sz, vp], i),
            "moe_sb_route_ffn_combine": ([vp, i, i, i, vp, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp], i),
            "moe_mx_expert_ffn_combine": ([vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, sz, vp], i),
            "moe_mx_route_ffn_combine": ([vp, i, i, i, vp, vp, i, i, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp], i),
            "moe_cpu_lane_create": ([i, ctypes.POINTER(vp)], i),
            "moe_cpu_lane_submit": ([vp, vp, i, i, i, vp, vp, u64p], i),
            "moe_cpu_lane_wait": ([vp, ctypes.c_uint64], i),
            "moe_cpu_lane_destroy": ([vp], i),
            "moe_cpu_lane_isa": ([], i),
            "moe_cpu_lane_force_isa": ([vp, i], i),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check_single_hip_runtime():
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line}
    if len(libs) > 1:
        raise MoEError(MOE_E_STATE, "load", f"two HIP runtimes are loaded: {sorted(libs)}")


def hip_runtime():
    """The HIP runtime shared with torch (for pinned host allocations)."""
    lib()
    return ctypes.CDLL("libamdhip64.so.7")


def _ptr(p):
    if p is None:
        return None
    if isinstance(p, int):
        return p
    if hasattr(p, "data_ptr"):
        return p.data_ptr()
    if hasattr(p, "ctypes"):  # numpy array (host memory)
        return p.ctypes.data
    raise TypeError(f"cannot pass {type(p)} as a pointer")


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # torch.cuda.Stream


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoEError(rc, where, lib().moe_last_error_message().decode())


# ----------------------------------------------------------------------- info
def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_last_hip_error() -> int:
    return lib().moe_last_hip_error()


def moe_last_error_message() -> str:
    return lib().moe_last_error_message().decode()


def moe_version() -> int:
    return lib().moe_version()


def moe_expert_bytes(hidden: int, inter: int) -> int:
    return lib().moe_expert_bytes(hidden, inter)


# ----------------------------------------------------------------------- router
def moe_router_workspace_bytes(T: int, E: int) -> int:
    return lib().moe_router_workspace_bytes(T, E)


def moe_router_topk(x, T, H, w_router, bias, E, k, topk_idx, topk_w, workspace, workspace_bytes, stream=None):
    _check(lib().moe_router_topk(_ptr(x), T, H, _ptr(w_router), _ptr(bias), E, k, _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(workspace), workspace_bytes, _stream(stream)), "moe_router_topk")


def moe_router_layers_workspace_bytes(n_layers: int, T: int, E: int) -> int:
    return lib().moe_router_layers_workspace_bytes(n_layers, T, E)


def moe_router_topk_layers(x, n_layers, T, H, w_router, bias, E, k, topk_idx, topk_w, workspace, workspace_bytes,
                           stream=None):
    _check(lib().moe_router_topk_layers(_ptr(x), n_layers, T, H, _ptr(w_router), _ptr(bias), E, k, _ptr(topk_idx),
                                        _ptr(topk_w), _ptr(workspace), workspace_bytes, _stream(stream)),
           "moe_router_topk_layers")


def moe_permute(topk_idx, T, k, E, count, offset, pair_of_row, stream=None):
    _check(lib().moe_permute(_ptr(topk_idx), T, k, E, _ptr(count), _ptr(offset), _ptr(pair_of_row),
                             _stream(stream)), "moe_permute")


# ----------------------------------------------------------------------- cache
def moe_cache_create(desc: moe_cache_desc, experts_host, slot_pool, expert_table, copy_stream) -> int:
    """experts_host: ctypes array / int address of L*E host pointers. Returns the cache handle."""
    out = ctypes.c_void_p()
    _check(lib().moe_cache_create(ctypes.byref(desc), _ptr(experts_host), _ptr(slot_pool), _ptr(expert_table),
                                  _stream(copy_stream), ctypes.byref(out)), "moe_cache_create")
    return out.value


def moe_cache_create_recording(desc: moe_cache_desc, slot_pool: int = 0, fail_copy_at: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(lib().moe_cache_create_recording(ctypes.byref(desc), slot_pool, fail_copy_at, ctypes.byref(out)),
           "moe_cache_create_recording")
    return out.value


def moe_cache_trace(cache: int):
    n = lib().moe_cache_trace(cache, None, 0)
    if n < 0:
        raise MoEError(MOE_E_STATE, "moe_cache_trace", "not a recording cache")
    buf = (ctypes.c_int64 * (4 * max(n, 1)))()
    lib().moe_cache_trace(cache, buf, n)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def _i32_array(values):
    arr = (ctypes.c_int32 * max(len(values), 1))()
    for j, v in enumerate(values):
        arr[j] = int(v)
    return arr


def moe_cache_lookup(cache: int, layer: int, experts):
    arr = _i32_array(experts)
    slots = (ctypes.c_int32 * max(len(experts), 1))()
    hits = ctypes.c_int()
    _check(lib().moe_cache_lookup(cache, layer, arr, len(experts), slots, ctypes.byref(hits)), "moe_cache_lookup")
    return [slots[j] for j in range(len(experts))], hits.value


def _i32_arg(values):
    """(pointer, count) of int32 expert ids: numpy int32 arrays pass through, other sequences are copied."""
    try:
        import numpy as np
        if isinstance(values, np.ndarray) and values.dtype == np.int32 and values.flags["C_CONTIGUOUS"]:
            return values, int(values.size)
    except ImportError:
        pass
    return _i32_array(values), len(values)


def moe_cache_prefetch(cache: int, layer: int, experts, compute_stream=None) -> int:
    arr, n_e = _i32_arg(experts)
    n = ctypes.c_int()
    _check(lib().moe_cache_prefetch(cache, layer, _ptr(arr) if hasattr(arr, "ctypes") else arr, n_e,
                                    _stream(compute_stream), ctypes.byref(n)), "moe_cache_prefetch")
    return n.value


def moe_cache_prefetch_async(cache: int, layer: int, experts) -> int:
    arr = _i32_array(experts)
    n = ctypes.c_int()
    _check(lib().moe_cache_prefetch_async(cache, layer, arr, len(experts), ctypes.byref(n)),
           "moe_cache_prefetch_async")
    return n.value


def moe_cache_split_copies(cache, second_copy_stream=None):
    _check(lib().moe_cache_split_copies(cache, _stream(second_copy_stream)), "moe_cache_split_copies")


def moe_cache_wait(cache: int, layer: int, compute_stream=None):
    _check(lib().moe_cache_wait(cache, layer, _stream(compute_stream)), "moe_cache_wait")


def moe_cache_release(cache: int, layer: int, compute_stream=None):
    _check(lib().moe_cache_release(cache, layer, _stream(compute_stream)), "moe_cache_release")


def moe_cache_stats(cache: int):
    h, m, b = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().moe_cache_stats(cache, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)), "moe_cache_stats")
    return h.value, m.value, b.value


def moe_cache_plan(cache: int, layer: int, ids, max_waves: int = 0, masks=None):
    """Waves of a layer's experts (see moe.h).  ids: host int32 numpy array (or a
    sequence) of the layer's top-k ids, repeats allowed; masks: optional host
    uint8 numpy array [max_waves, E] that the call fills.  Returns the waves as
    lists of expert ids."""
    import numpy as np
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
    n = int(ids.size)
    if masks is not None:
        assert masks.dtype == np.uint8 and masks.flags["C_CONTIGUOUS"] and masks.ndim == 2
        max_waves = masks.shape[0]
    max_waves = max_waves or max(n, 1)
    experts = np.empty(max(n, 1), np.int32)
    starts = np.empty(max_waves + 1, np.int32)
    nw = ctypes.c_int()
    _check(lib().moe_cache_plan(cache, layer, ids.ctypes.data if n else None, n, experts.ctypes.data,
                                starts.ctypes.data, max_waves, None if masks is None else masks.ctypes.data,
                                ctypes.byref(nw)), "moe_cache_plan")
    return [experts[starts[v]:starts[v + 1]].tolist() for v in range(nw.value)]


def moe_cache_copy_timing(cache: int, enable: bool):
    _check(lib().moe_cache_copy_timing(cache, int(bool(enable))), "moe_cache_copy_timing")


def moe_cache_copy_busy(cache: int):
    """-> (busy_ms, span_ms, n_copies) over the copies timed so far (blocks)."""
    b, sp, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_uint64()
    _check(lib().moe_cache_copy_busy(cache, ctypes.byref(b), ctypes.byref(sp), ctypes.byref(n)),
           "moe_cache_copy_busy")
    return b.value, sp.value, n.value


def moe_cache_plan_step(cache: int, ids, ids_per_layer: int, wave_experts, wave_start, max_waves: int, masks,
                        n_waves, issue_single: bool = True) -> int:
    """moe_cache_plan for every layer (see moe.h); all arrays are caller-owned host
    numpy arrays (ids and outputs int32, masks uint8 or None).  Returns the number
    of misses streamed for single-wave layers."""
    nc = ctypes.c_int()
    _check(lib().moe_cache_plan_step(cache, _ptr(ids), ids_per_layer, _ptr(wave_experts), _ptr(wave_start),
                                     max_waves, _ptr(masks), _ptr(n_waves), int(bool(issue_single)),
                                     ctypes.byref(nc)), "moe_cache_plan_step")
    return nc.value


def moe_cache_reset(cache: int):
    _check(lib().moe_cache_reset(cache), "moe_cache_reset")


def moe_cache_destroy(cache: int):
    lib().moe_cache_destroy(cache)


# ----------------------------------------------------------------------- FFN
def moe_expert_ffn_workspace_bytes(T, H, I, E, k, has_shared) -> int:
    return lib().moe_expert_ffn_workspace_bytes(T, H, I, E, k, int(bool(has_shared)))


def moe_expert_ffn(x, T, H, I, E, topk_idx, k, expert_table, shared_slab, expert_mask, y, workspace,
                   workspace_bytes, path=MOE_FFN_AUTO, stream=None):
    _check(lib().moe_expert_ffn(_ptr(x), T, H, I, E, _ptr(topk_idx), k, _ptr(expert_table), _ptr(shared_slab),
                                _ptr(expert_mask), _ptr(y), _ptr(workspace), workspace_bytes, path,
                                _stream(stream)), "moe_expert_ffn")


def moe_expert_gate_up(x, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                       expert_mask, h, path=MOE_FFN_AUTO, stream=None):
    _check(lib().moe_expert_gate_up(_ptr(x), T, H, I, E, _ptr(topk_idx), k, _ptr(count), _ptr(offset),
                                    _ptr(pair_of_row), _ptr(expert_table), _ptr(shared_slab), _ptr(expert_mask),
                                    _ptr(h), path, _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(h, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                    expert_mask, y, path=MOE_FFN_AUTO, stream=None):
    _check(lib().moe_expert_down(_ptr(h), T, H, I, E, _ptr(topk_idx), k, _ptr(count), _ptr(offset),
                                 _ptr(pair_of_row), _ptr(expert_table), _ptr(shared_slab), _ptr(expert_mask),
                                 _ptr(y), path, _stream(stream)), "moe_expert_down")


def moe_expert_ffn_fmt(x, T, H, I, E, topk_idx, k, expert_table, shared_slab, expert_mask, y, workspace,
                       workspace_bytes, path=MOE_FFN_AUTO, format=0, stream=None):
    _check(lib().moe_expert_ffn_fmt(_ptr(x), T, H, I, E, _ptr(topk_idx), k, _ptr(expert_table), _ptr(shared_slab),
                                    _ptr(expert_mask), _ptr(y), _ptr(workspace), workspace_bytes, path, format,
                                    _stream(stream)), "moe_expert_ffn_fmt")


def moe_expert_gate_up_fmt(x, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                           expert_mask, h, path=MOE_FFN_AUTO, format=0, stream=None):
    _check(lib().moe_expert_gate_up_fmt(_ptr(x), T, H, I, E, _ptr(topk_idx), k, _ptr(count), _ptr(offset),
                                        _ptr(pair_of_row), _ptr(expert_table), _ptr(shared_slab),
                                        _ptr(expert_mask), _ptr(h), path, format, _stream(stream)),
           "moe_expert_gate_up_fmt")


def moe_expert_down_fmt(h, T, H, I, E, topk_idx, k, count, offset, pair_of_row, expert_table, shared_slab,
                        expert_mask, y, path=MOE_FFN_AUTO, format=0, stream=None):
    _check(lib().moe_expert_down_fmt(_ptr(h), T, H, I, E, _ptr(topk_idx), k, _ptr(count), _ptr(offset),
                                     _ptr(pair_of_row), _ptr(expert_table), _ptr(shared_slab), _ptr(expert_mask),
                                     _ptr(y), path, format, _stream(stream)), "moe_expert_down_fmt")


def moe_quant_act_mx(x, rows, K, out, scales, stream=None):
    _check(lib().moe_quant_act_mx(_ptr(x), rows, K, _ptr(out), _ptr(scales), _stream(stream)), "moe_quant_act_mx")


def moe_expert_ffn_combine(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, workspace,
                           workspace_bytes, path=MOE_FFN_AUTO, stream=None):
    _check(lib().moe_expert_ffn_combine(_ptr(x), T, H, I, E, _ptr(topk_idx), _ptr(topk_w), k, _ptr(expert_table),
                                        _ptr(shared_slab), _ptr(out), _ptr(workspace), workspace_bytes, path,
                                        _stream(stream)), "moe_expert_ffn_combine")


def moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, has_shared) -> int:
    return lib().moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, int(bool(has_shared)))


def moe_route_ffn_combine(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w, out,
                          workspace, workspace_bytes, stream=None, prefetch=None, prefetch_bytes=0):
    _check(lib().moe_route_ffn_combine(_ptr(x), T, H, I, _ptr(w_router), _ptr(bias), E, k, _ptr(expert_table),
                                       _ptr(shared_slab), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(workspace),
                                       workspace_bytes, _ptr(prefetch), prefetch_bytes, _stream(stream)),
           "moe_route_ffn_combine")


def moe_noalloc_scratch_bytes() -> int:
    return lib().moe_noalloc_scratch_bytes()


def moe_route_ffn_combine_noalloc(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w,
                                  out, stream=None, prefetch=None, prefetch_bytes=0):
    _check(lib().moe_route_ffn_combine_noalloc(_ptr(x), T, H, I, _ptr(w_router), _ptr(bias), E, k,
                                               _ptr(expert_table), _ptr(shared_slab), _ptr(topk_idx), _ptr(topk_w),
                                               _ptr(out), _ptr(prefetch), prefetch_bytes, _stream(stream)),
           "moe_route_ffn_combine_noalloc")


def moe_combine(y, topk_w, T, k, H, has_shared, out, stream=None):
    _check(lib().moe_combine(_ptr(y), _ptr(topk_w), T, k, H, int(bool(has_shared)), _ptr(out), _stream(stream)),
           "moe_combine")


def moe_scatter_rows(src, rows, n, H, dst, stream=None):
    _check(lib().moe_scatter_rows(_ptr(src), _ptr(rows), n, H, _ptr(dst), _stream(stream)), "moe_scatter_rows")


def moe_residual_norm(add, resid, T, H, eps, x_next, stream=None):
    _check(lib().moe_residual_norm(_ptr(add) if add is not None else None, _ptr(resid), T, H, float(eps),
                                   _ptr(x_next), _stream(stream)), "moe_residual_norm")


def moe_debug_dequant(slab, H, I, which, out, stream=None):
    _check(lib().moe_debug_dequant(_ptr(slab), H, I, which, _ptr(out), _stream(stream)), "moe_debug_dequant")


# ----------------------------------------------------------------------- CPU lane
def moe_cpu_lane_create(threads: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().moe_cpu_lane_create(int(threads), ctypes.byref(out)), "moe_cpu_lane_create")
    return out.value


def moe_cpu_lane_submit(lane, slab, H, I, M, x_rows, y_rows) -> int:
    """x_rows / y_rows: sequences of M host addresses (bf16 rows in, fp32 rows out).
    Returns the job's ticket."""
    xs = (ctypes.c_void_p * max(M, 1))(*[int(a) for a in x_rows])
    ys = (ctypes.c_void_p * max(M, 1))(*[int(a) for a in y_rows])
    t = ctypes.c_uint64()
    _check(lib().moe_cpu_lane_submit(lane, _ptr(slab), H, I, M, xs, ys, ctypes.byref(t)), "moe_cpu_lane_submit")
    return t.value


def moe_cpu_lane_wait(lane, ticket: int):
    _check(lib().moe_cpu_lane_wait(lane, ticket), "moe_cpu_lane_wait")


def moe_cpu_lane_destroy(lane):
    _check(lib().moe_cpu_lane_destroy(lane), "moe_cpu_lane_destroy")


def moe_cpu_lane_isa() -> int:
    return lib().moe_cpu_lane_isa()


def moe_cpu_lane_force_isa(lane, isa: int):
    _check(lib().moe_cpu_lane_force_isa(lane, isa), "moe_cpu_lane_force_isa")


# ----------------------------------------------------------------------- MXFP4 weights
def moe_expert_bytes_mx(H: int, I: int) -> int:
    return lib().moe_expert_bytes_mx(H, I)


def moe_mx_expert_ffn_combine(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, workspace,
                              workspace_bytes, stream=None):
    _check(lib().moe_mx_expert_ffn_combine(_ptr(x), T, H, I, E, _ptr(topk_idx), _ptr(topk_w), k, _ptr(expert_table),
                                           _ptr(shared_slab), _ptr(out), _ptr(workspace), workspace_bytes,
                                           _stream(stream)), "moe_mx_expert_ffn_combine")


def moe_mx_route_ffn_combine(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w, out,
                             workspace, workspace_bytes, stream=None, prefetch=None, prefetch_bytes=0):
    _check(lib().moe_mx_route_ffn_combine(_ptr(x), T, H, I, _ptr(w_router), _ptr(bias), E, k, _ptr(expert_table),
                                          _ptr(shared_slab), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(workspace),
                                          workspace_bytes, _ptr(prefetch), prefetch_bytes, _stream(stream)),
           "moe_mx_route_ffn_combine")


# ----------------------------------------------------------------------- super-block weights
def moe_expert_bytes_sb(H: int, I: int) -> int:
    return lib().moe_expert_bytes_sb(H, I)


def moe_sb_expert_ffn_combine(x, T, H, I, E, topk_idx, topk_w, k, expert_table, shared_slab, out, workspace,
                              workspace_bytes, stream=None):
    _check(lib().moe_sb_expert_ffn_combine(_ptr(x), T, H, I, E, _ptr(topk_idx), _ptr(topk_w), k, _ptr(expert_table),
                                           _ptr(shared_slab), _ptr(out), _ptr(workspace), workspace_bytes,
                                           _stream(stream)), "moe_sb_expert_ffn_combine")


def moe_sb_route_ffn_combine(x, T, H, I, w_router, bias, E, k, expert_table, shared_slab, topk_idx, topk_w, out,
                             workspace, workspace_bytes, stream=None, prefetch=None, prefetch_bytes=0):
    _check(lib().moe_sb_route_ffn_combine(_ptr(x), T, H, I, _ptr(w_router), _ptr(bias), E, k, _ptr(expert_table),
                                          _ptr(shared_slab), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(workspace),
                                          workspace_bytes, _ptr(prefetch), prefetch_bytes, _stream(stream)),
           "moe_sb_route_ffn_combine")
