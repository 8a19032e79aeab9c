"""ctypes binding of the C ABI in include/qtip_moe.h (argument marshalling only).

Every function keeps its C name.  Pointer arguments accept an int address, None (NULL)
or any object with a `data_ptr()` method (a torch tensor); device memory and streams
come from PyTorch, all computation happens in the HIP library.  The binding never
falls back to anything else: if the library is missing, `lib()` raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libqtip_moe.so"
LIB_PATH = os.path.join(_HERE, LIB_NAME)

QTIP_OK = 0
QTIP_ERR_INVALID_ARG = 1
QTIP_ERR_INVALID_CONFIG = 2
QTIP_ERR_NOT_SUPPORTED = 3
QTIP_ERR_HIP = 4
QTIP_ERR_CAPTURING = 5

QTIP_ARM_AUTO = 0
QTIP_ARM_GEMV = 1
QTIP_ARM_GROUPED = 2
QTIP_ARM_DEQUANT = 3
QTIP_ACT_AUTO = 0
QTIP_ACT_ROWS = 1
QTIP_ACT_FRAGMENTS = 2
QTIP_OUT_BF16 = 0
QTIP_OUT_F32 = 1
QTIP_DEFAULT_DECODE_FLOOR_BITSHIFT = 7
QTIP_DEFAULT_DECODE_FLOOR_LUT = 4
QTIP_DECODE_REGIME_MAX_TOKENS = 8
QTIP_RUNG_BITSHIFT = 0
QTIP_RUNG_LUT = 1
QTIP_SMALL_BATCH_FUSED = 0
QTIP_SMALL_BATCH_SEPARATE = 1
QTIP_LUT_RUNG_BITS = 9


class qtip_moe_desc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("arm_override", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("dispatch_tile_m", ctypes.c_int32), ("dequant_traffic_ratio", ctypes.c_int32),
                ("act_layout", ctypes.c_int32), ("rung", ctypes.c_int32), ("decode_floor", ctypes.c_int32),
                ("small_batch", ctypes.c_int32)]


class qtip_moe_weights(ctypes.Structure):
    _fields_ = [("codes_gate", ctypes.c_void_p), ("codes_up", ctypes.c_void_p), ("codes_down", ctypes.c_void_p),
                ("scale_gate", ctypes.c_void_p), ("scale_up", ctypes.c_void_p), ("scale_down", ctypes.c_void_p),
                ("lut", ctypes.c_void_p)]


QTIP_VARIANT_SLOTS = 12


class qtip_moe_stats_t(ctypes.Structure):
    _fields_ = [("forward_calls", ctypes.c_uint64), ("gemv_launches", ctypes.c_uint64),
                ("grouped_launches", ctypes.c_uint64), ("route_launches", ctypes.c_uint64),
                ("combine_launches", ctypes.c_uint64), ("router_launches", ctypes.c_uint64),
                ("dequant_launches", ctypes.c_uint64),
                ("last_arm", ctypes.c_int32),
                ("last_n_tokens", ctypes.c_int32),
                ("gemv_variant_launches", ctypes.c_uint64 * QTIP_VARIANT_SLOTS),
                ("grouped_variant_launches", ctypes.c_uint64 * QTIP_VARIANT_SLOTS),
                ("routed_in_gate_up", ctypes.c_uint64), ("combined_in_down", ctypes.c_uint64)]


class qtip_moe_kernel_shape(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("waves_per_workgroup", ctypes.c_int32),
                ("rows_per_task", ctypes.c_int32), ("pairs_per_decode", ctypes.c_int32)]


class qtip_moe_schedule(ctypes.Structure):
    _fields_ = [("arm", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("gate_up", qtip_moe_kernel_shape),
                ("down", qtip_moe_kernel_shape), ("route_in_gate_up", ctypes.c_int32),
                ("combine_in_down", ctypes.c_int32)]


class QtipError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} -> {status_name(status)}: {detail}")


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "qtip_moe_plan": (_I32, [ctypes.POINTER(qtip_moe_desc), ctypes.c_int, ctypes.POINTER(_P)]),
    "qtip_moe_plan_for_arch": (_I32, [ctypes.POINTER(qtip_moe_desc), ctypes.c_char_p, ctypes.POINTER(_P)]),
    "qtip_moe_plan_destroy": (_I32, [_P]),
    "qtip_moe_plan_info": (_I32, [_P, ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_I32)]),
    "qtip_moe_select_arm": (_I32, [_P, _I32]),
    "qtip_moe_select_grouped": (_I32, [_P, _I32]),
    "qtip_moe_plan_schedule": (_I32, [_P, _I32, ctypes.POINTER(qtip_moe_schedule)]),
    "qtip_fill_woken_experts": (ctypes.c_double, [_I32, _I32, _I32]),
    "qtip_fill_pairs_per_woken_expert": (ctypes.c_double, [_I32, _I32, _I32]),
    "qtip_fill_select_grouped": (_I32, [_I32, _I32, _I32, _I32]),
    "qtip_fill_min_tokens": (_I32, [_I32, _I32, _I32]),
    "qtip_moe_forward": (_I32, [_P, ctypes.POINTER(qtip_moe_weights), _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
    "qtip_moe_forward_noalloc": (_I32, [_P, ctypes.POINTER(qtip_moe_weights), _P, _P, _I32, _P, _P]),
    "qtip_moe_forward_hidden": (_I32, [_P, ctypes.POINTER(qtip_moe_weights), _P, _P, _I32, _P, _P, ctypes.c_size_t,
                                       _P]),
    "qtip_moe_router_logits": (_I32, [_P, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
    "qtip_moe_router_split": (_I32, [_P, _I32]),
    "qtip_moe_dequant_range": (_I32, [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "qtip_moe_dequantize": (_I32, [_P, ctypes.POINTER(qtip_moe_weights), _I32, _I32, _P, _P]),
    "qtip_fill_select_arm": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "qtip_moe_route": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "qtip_expert_matmul": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _I32, _P, _P]),
    "qtip_moe_stats": (_I32, [_P, ctypes.POINTER(qtip_moe_stats_t)]),
    "qtip_moe_stats_reset": (_I32, [_P]),
    "qtip_moe_engaged_line": (_I32, [_P, _I32, ctypes.c_char_p, ctypes.c_size_t]),
    "qtip_moe_log_engaged": (_I32, [_P, _I32, ctypes.POINTER(_I32)]),
    "qtip_arch_witness": (_I32, [ctypes.c_int, _P]),
    "qtip_moe_profile_enable": (_I32, [_P, _I32]),
    "qtip_moe_profile_read": (_I32, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)]),
    "qtip_measure_lut_gather": (_I32, [_I32, _P, ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_double)]),
    "qtip_status_string": (ctypes.c_char_p, [_I32]),
    "qtip_last_error_detail": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -m "
                              f"trellis_quantized_moe_expert_amd.build or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_name(status: int) -> str:
    return lib().qtip_status_string(status).decode()


def last_error_detail() -> str:
    return lib().qtip_last_error_detail().decode()


def _ptr(obj):
    if obj is None:
        return None
    if hasattr(obj, "data_ptr"):
        return obj.data_ptr()
    return int(obj)


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, status: int):
    if status != QTIP_OK:
        raise QtipError(fn, status, last_error_detail())


def make_desc(num_experts, top_k, hidden, inter, max_tokens, arm_override=QTIP_ARM_AUTO, variant=0,
              out_dtype=QTIP_OUT_F32, tile_m=0, dispatch_tile_m=0, dequant_traffic_ratio=0,
              act_layout=QTIP_ACT_AUTO, rung=QTIP_RUNG_BITSHIFT, decode_floor=0,
              small_batch=QTIP_SMALL_BATCH_FUSED) -> qtip_moe_desc:
    return qtip_moe_desc(num_experts, top_k, hidden, inter, max_tokens, arm_override, variant, out_dtype, tile_m,
                         dispatch_tile_m, dequant_traffic_ratio, act_layout, rung, decode_floor, small_batch)


def make_weights(codes_gate, codes_up, codes_down, scale_gate, scale_up, scale_down, lut) -> qtip_moe_weights:
    return qtip_moe_weights(*(_ptr(a) for a in (codes_gate, codes_up, codes_down, scale_gate, scale_up,
                                                scale_down, lut)))


# ---- the C entry points, same names --------------------------------------------------------
def qtip_moe_plan(desc: qtip_moe_desc, device: int = 0) -> int:
    out = _P()
    _check("qtip_moe_plan", lib().qtip_moe_plan(ctypes.byref(desc), device, ctypes.byref(out)))
    return out.value


def qtip_moe_plan_for_arch(desc: qtip_moe_desc, arch: str) -> int:
    out = _P()
    _check("qtip_moe_plan_for_arch", lib().qtip_moe_plan_for_arch(ctypes.byref(desc), arch.encode(), ctypes.byref(out)))
    return out.value


def qtip_moe_plan_destroy(plan: int) -> None:
    _check("qtip_moe_plan_destroy", lib().qtip_moe_plan_destroy(plan))


def qtip_moe_plan_info(plan: int) -> dict:
    tm, mt, ws = _I32(), _I32(), ctypes.c_size_t()
    _check("qtip_moe_plan_info", lib().qtip_moe_plan_info(plan, ctypes.byref(tm), ctypes.byref(ws), ctypes.byref(mt)))
    return {"tile_m": tm.value, "workspace_bytes": ws.value, "min_tokens_grouped": mt.value}


def qtip_moe_plan_schedule(plan: int, n_tokens: int) -> dict:
    out = qtip_moe_schedule()
    _check("qtip_moe_plan_schedule", lib().qtip_moe_plan_schedule(plan, n_tokens, ctypes.byref(out)))
    shape = lambda sh: {name: getattr(sh, name) for name, _ in qtip_moe_kernel_shape._fields_}
    return {"arm": out.arm, "tile_m": out.tile_m, "gate_up": shape(out.gate_up), "down": shape(out.down),
            "route_in_gate_up": out.route_in_gate_up, "combine_in_down": out.combine_in_down}


def qtip_moe_select_arm(plan: int, n_tokens: int) -> int:
    return lib().qtip_moe_select_arm(plan, n_tokens)


def qtip_moe_select_grouped(plan: int, n_tokens: int) -> int:
    return lib().qtip_moe_select_grouped(plan, n_tokens)


def qtip_fill_woken_experts(n, k, E) -> float:
    return lib().qtip_fill_woken_experts(n, k, E)


def qtip_fill_pairs_per_woken_expert(n, k, E) -> float:
    return lib().qtip_fill_pairs_per_woken_expert(n, k, E)


def qtip_fill_select_grouped(n, k, E, tile_m) -> int:
    return lib().qtip_fill_select_grouped(n, k, E, tile_m)


def qtip_fill_min_tokens(k, E, tile_m) -> int:
    return lib().qtip_fill_min_tokens(k, E, tile_m)


def qtip_moe_forward(plan, weights: qtip_moe_weights, x_bf16, logits, n_tokens, out, workspace, workspace_bytes,
                     stream=None) -> None:
    _check("qtip_moe_forward", lib().qtip_moe_forward(plan, ctypes.byref(weights), _ptr(x_bf16), _ptr(logits),
                                                      n_tokens, _ptr(out), _ptr(workspace), workspace_bytes,
                                                      _stream(stream)))


QTIP_NOALLOC_SCRATCH_BYTES = 64 << 20


def qtip_moe_forward_noalloc(plan, weights: qtip_moe_weights, x_bf16, logits, n_tokens, out, stream=None) -> None:
    _check("qtip_moe_forward_noalloc", lib().qtip_moe_forward_noalloc(plan, ctypes.byref(weights), _ptr(x_bf16),
                                                                      _ptr(logits), n_tokens, _ptr(out),
                                                                      _stream(stream)))


def qtip_moe_forward_hidden(plan, weights: qtip_moe_weights, w_router_bf16, x_bf16, n_tokens, out, workspace,
                            workspace_bytes, stream=None) -> None:
    _check("qtip_moe_forward_hidden", lib().qtip_moe_forward_hidden(plan, ctypes.byref(weights), _ptr(w_router_bf16),
                                                                    _ptr(x_bf16), n_tokens, _ptr(out),
                                                                    _ptr(workspace), workspace_bytes,
                                                                    _stream(stream)))


def qtip_moe_router_logits(plan, x_bf16, w_router_bf16, n_tokens, logits, workspace, workspace_bytes,
                           stream=None) -> None:
    _check("qtip_moe_router_logits", lib().qtip_moe_router_logits(plan, _ptr(x_bf16), _ptr(w_router_bf16), n_tokens,
                                                                  _ptr(logits), _ptr(workspace), workspace_bytes,
                                                                  _stream(stream)))


def qtip_moe_dequant_range(plan) -> tuple:
    lo, hi = _I32(), _I32()
    _check("qtip_moe_dequant_range", lib().qtip_moe_dequant_range(plan, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def qtip_moe_dequantize(plan, weights: qtip_moe_weights, matrix, expert, dense_out, stream=None) -> None:
    _check("qtip_moe_dequantize", lib().qtip_moe_dequantize(plan, ctypes.byref(weights), matrix, expert,
                                                            _ptr(dense_out), _stream(stream)))


def qtip_fill_select_arm(n, k, E, tile_m, dequant_ratio) -> int:
    return lib().qtip_fill_select_arm(n, k, E, tile_m, dequant_ratio)


def qtip_moe_router_split(plan, n_tokens) -> int:
    return lib().qtip_moe_router_split(plan, n_tokens)


def qtip_moe_route(plan, logits, n_tokens, topk_idx, topk_w, counts, offsets, sorted_pair, tile_map, n_tiles,
                   stream=None) -> None:
    _check("qtip_moe_route", lib().qtip_moe_route(plan, _ptr(logits), n_tokens, _ptr(topk_idx), _ptr(topk_w),
                                                  _ptr(counts), _ptr(offsets), _ptr(sorted_pair), _ptr(tile_map),
                                                  _ptr(n_tiles), _stream(stream)))


def qtip_expert_matmul(plan, arm, codes, scales, lut, num_experts, rows, cols, a_bf16, n_rows_a, unit_map, n_units,
                       y, stream=None) -> None:
    _check("qtip_expert_matmul", lib().qtip_expert_matmul(plan, arm, _ptr(codes), _ptr(scales), _ptr(lut),
                                                          num_experts, rows, cols, _ptr(a_bf16), n_rows_a,
                                                          _ptr(unit_map), n_units, _ptr(y), _stream(stream)))


def qtip_moe_stats(plan) -> dict:
    s = qtip_moe_stats_t()
    _check("qtip_moe_stats", lib().qtip_moe_stats(plan, ctypes.byref(s)))
    out = {}
    for name, _ in qtip_moe_stats_t._fields_:
        v = getattr(s, name)
        out[name] = list(v) if isinstance(v, ctypes.Array) else v
    return out


def qtip_moe_stats_reset(plan) -> None:
    _check("qtip_moe_stats_reset", lib().qtip_moe_stats_reset(plan))


def qtip_moe_engaged_line(plan, n_tokens) -> str:
    buf = ctypes.create_string_buffer(512)
    _check("qtip_moe_engaged_line", lib().qtip_moe_engaged_line(plan, n_tokens, buf, len(buf)))
    return buf.value.decode()


def qtip_moe_log_engaged(plan, n_tokens) -> bool:
    printed = _I32()
    _check("qtip_moe_log_engaged", lib().qtip_moe_log_engaged(plan, n_tokens, ctypes.byref(printed)))
    return bool(printed.value)


def qtip_arch_witness(device: int = 0, stream=None) -> None:
    _check("qtip_arch_witness", lib().qtip_arch_witness(device, _stream(stream)))


PROFILE_STAGES = ("route", "bin", "gate_up", "down", "combine")


def qtip_moe_profile_enable(plan, capacity: int) -> None:
    _check("qtip_moe_profile_enable", lib().qtip_moe_profile_enable(plan, capacity))


def qtip_moe_profile_read(plan) -> dict:
    ms = (ctypes.c_double * 5)()
    n = _I32()
    _check("qtip_moe_profile_read", lib().qtip_moe_profile_read(plan, ms, ctypes.byref(n)))
    return {"n_forwards": n.value, **{name: ms[i] for i, name in enumerate(PROFILE_STAGES)}}


def qtip_measure_lut_gather(rounds: int, sink, sink_elems: int, stream=None) -> float:
    out = ctypes.c_double()
    _check("qtip_measure_lut_gather", lib().qtip_measure_lut_gather(rounds, _ptr(sink), sink_elems, _stream(stream),
                                                                    ctypes.byref(out)))
    return out.value


def raw_status(fn_name: str, *args) -> int:
    """Call a C entry point with raw arguments and return its status (for error-path tests)."""
    return getattr(lib(), fn_name)(*args)
